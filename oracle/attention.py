"""Block-causal chunk attention over the ring cache (oracle, float64).

Test infrastructure only (see ``oracle/__init__.py``).

Definition (readings of the pages, one per line):
* Every new query attends over every cached slot, history plus its own
  chunk (Runway Characters, abstract: each call reads the whole cache).
* Block-causal mask: a query of block b sees the slots whose block id is
  <= b; inside its own block it sees everything, across blocks only the past
  ("Why Live Video Generation Still Struggles With Timing", transcript on
  streaming editors; StreamLTX project page, Training: causal masks on all
  paths so nothing reads the future).  Slots with block id -1 were never
  written and are invisible.
* Cache bias: an additive term on the scaled logit of every visible slot of
  an EARLIER block; the query's own block gets none (video-conductor,
  "Plastic Windows": the cache attention bias is lowered during prompt
  transitions and restored afterwards).
* Queries are rotated by their positions with the same RoPE as the keys.

For query i: pos_i = q_pos0 + i, b_i = q_block0 + floor(i / q_block_len),
    q'_i   = RoPE(q_i, pos_i)
    l_is   = sigma * (q'_i . k_s) + beta * [blk_s < b_i]   for visible s
    out_i  = sum_s softmax_s(l_is) v_s,   lse_i = ln sum_s exp(l_is)
sigma = softmax_scale, or 1/sqrt(d) when 0 is given.  A query with no
visible slot gets out = 0 and lse = -inf.

Two generalisations serve the joint audio-video block (StreamLTX project
page, Training and Data):
* per-query blocks: b_i may be given for every query (the first block of a
  take carries one latent frame more than the others -- 4 + 3k video and
  26 + 25k audio frames -- so blocks of queries are not all one length);
* the same-block mask for the text cross-attention paths: each block sees
  only the prompt of its own segment.  The text slots carry their segment's
  id as block id, each query its block's segment id, and slot s is visible
  to query i iff blk_s == b_i (no bias: the prompt is not history).
"""
from __future__ import annotations

import numpy as np

from .rope import rope


def query_blocks(n_q: int, q_block0: int, q_block_len: int) -> np.ndarray:
    return q_block0 + np.arange(n_q) // q_block_len


def visibility(slot_block: np.ndarray, qblk: np.ndarray, mask: str = "causal"
               ) -> tuple[np.ndarray, np.ndarray]:
    """(visible, earlier_block) boolean masks of shape [n_q][N].
    mask "causal": visible iff blk != -1 and blk <= b_i, bias on blk < b_i;
    mask "same": visible iff blk == b_i (>= 0), never biased."""
    blk = np.asarray(slot_block)[None, :]
    qb = np.asarray(qblk)[:, None]
    if mask == "same":
        vis = (blk != -1) & (blk == qb)
        return vis, np.zeros_like(vis)
    if mask != "causal":
        raise ValueError(mask)
    vis = (blk != -1) & (blk <= qb)
    earlier = vis & (blk < qb)
    return vis, earlier


def chunk_attention(k_vals: np.ndarray, v_vals: np.ndarray, slot_block: np.ndarray,
                    q: np.ndarray, q_pos0: int, q_block0: int, q_block_len: int,
                    cache_bias: float, softmax_scale: float, rope_base: float,
                    q_blocks=None, mask: str = "causal"):
    """k_vals, v_vals: float64 [H][N][d]; q: float64 [n_q][H][d] (unrotated).
    q_blocks: optional [n_q] block ids (then q_block0 and q_block_len are
    not used); mask: "causal" or "same".

    Returns (out float64 [n_q][H][d], lse float64 [H][n_q])."""
    H, N, d = k_vals.shape
    n_q = q.shape[0]
    sigma = softmax_scale if softmax_scale != 0 else 1.0 / np.sqrt(d)
    pos = q_pos0 + np.arange(n_q)
    qr = rope(q, pos[:, None], rope_base)
    qblk = (query_blocks(n_q, q_block0, q_block_len) if q_blocks is None
            else np.asarray(q_blocks, dtype=np.int64))
    vis, earlier = visibility(slot_block, qblk, mask)
    bias = np.where(earlier, float(cache_bias), 0.0)
    any_vis = vis.any(axis=1)
    out = np.zeros((n_q, H, d), dtype=np.float64)
    lse = np.full((H, n_q), -np.inf, dtype=np.float64)
    for h in range(H):
        logits = sigma * (qr[:, h, :] @ k_vals[h].T) + bias
        logits = np.where(vis, logits, -np.inf)
        m = np.max(logits, axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(logits - m)
        l = p.sum(axis=1, keepdims=True)
        safe_l = np.where(l > 0, l, 1.0)
        out[:, h, :] = np.where(any_vis[:, None], (p @ v_vals[h]) / safe_l, 0.0)
        lse[h] = np.where(any_vis, m[:, 0] + np.log(safe_l[:, 0]), -np.inf)
    return out, lse


def ring_attention(ring, q, q_pos0, q_block0, q_block_len, cache_bias, softmax_scale=0.0,
                   q_blocks=None, mask="causal"):
    """chunk_attention over an oracle Ring."""
    return chunk_attention(ring.k_values(), ring.v_values(), ring.slot_block, q,
                           q_pos0, q_block0, q_block_len, cache_bias, softmax_scale,
                           ring.rope_base, q_blocks=q_blocks, mask=mask)
