"""Scored content memory: per-key attention mass and the top-M selection
(oracle, float64).

Test infrastructure only (see ``oracle/__init__.py``).

StreamLTX project page, "Why a long take does not slow down": long-context
KV is split into an anchor, a content memory and a FIFO of recent blocks;
each layer scores its own keys on attention quality and temporal diversity
and evicts down to a top-M budget.  The page gives no formula; the plainest
reading taken here:

* Attention quality of a cached key = the attention mass it receives, the
  column sum over queries of the softmax probabilities of the attention that
  reads it (``key_mass``), per head; a slot's score is the sum over heads
  (a slot holds one token for every head of the layer, so heads keep or
  drop it together).
* Temporal diversity = diminishing returns inside one block (one chunk of
  time): the memory maximises  sum over blocks b of
  sum_k  Q_b,(k) * gamma^k,  where Q_b,(0) >= Q_b,(1) >= ... are the scores
  of the tokens it keeps from block b and gamma in (0, 1] is the diversity
  weight.  gamma = 1 is plain top-M by score; a smaller gamma spreads the
  memory over more blocks.
* The candidates are the tokens already in the memory plus the history
  tokens the next write pushes out of the FIFO; min(M, #candidates) of them
  are kept (``select_memory``).

The selection is the greedy rule on that objective: every block offers its
best remaining token (largest Q, ties to the smaller slot), whose gain is
Q_s * gamma^c with c the tokens already taken from that block; the largest
gain is taken, ties to the smaller c, then to the smaller slot.  The
objective is separable and concave per block, so the greedy picks are an
optimal set (the tests check this against brute force over all subsets on
small cases).  Precision fixed so that the choice is reproducible: Q_s is
the float64 sum of the float32 per-head scores in head order 0..H-1;
gamma^c is the float32 product gamma * gamma * ... (c factors, left to
right, each product rounded to float32), gamma^0 = 1, gamma the float32
value given; the gain is the float64 product of Q_s and gamma^c.  A float32
chain never increases with c (each rounding is monotone), which keeps every
block's gains in order.  Scores are finite and non-negative (attention mass
is).
"""
from __future__ import annotations

import numpy as np

from .attention import query_blocks, visibility
from .rope import rope


def key_mass(k_vals: np.ndarray, slot_block: np.ndarray, q: np.ndarray, q_pos0: int,
             q_block0: int, q_block_len: int, cache_bias: float, softmax_scale: float,
             rope_base: float) -> np.ndarray:
    """Attention mass per head and slot, float64 [H][N]:
    mass[h][s] = sum_i p_h(i, s), p the block-causal softmax of
    ``oracle.attention.chunk_attention`` (same logits, same mask and bias).
    Invisible slots get 0; a query that sees no slot adds nothing."""
    H, N, d = k_vals.shape
    n_q = q.shape[0]
    sigma = softmax_scale if softmax_scale != 0 else 1.0 / np.sqrt(d)
    qr = rope(q, (q_pos0 + np.arange(n_q))[:, None], rope_base)
    vis, earlier = visibility(slot_block, query_blocks(n_q, q_block0, q_block_len))
    bias = np.where(earlier, float(cache_bias), 0.0)
    mass = np.zeros((H, N), dtype=np.float64)
    for h in range(H):
        logits = np.where(vis, sigma * (qr[:, h, :] @ k_vals[h].T) + bias, -np.inf)
        m = np.max(logits, axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(logits - m)
        z = p.sum(axis=1, keepdims=True)
        p = p / np.where(z > 0, z, 1.0)
        mass[h] = p.sum(axis=0)
    return mass


def ring_key_mass(ring, q, q_pos0, q_block0, q_block_len, cache_bias, softmax_scale=0.0):
    """key_mass over an oracle Ring."""
    return key_mass(ring.k_values(), ring.slot_block, q, q_pos0, q_block0, q_block_len,
                    cache_bias, softmax_scale, ring.rope_base)


def slot_score(key_score: np.ndarray, s: int) -> float:
    """Q_s: float64 sum over heads, in head order, of the float32 scores."""
    total = 0.0
    for h in range(key_score.shape[0]):
        total += float(np.float32(key_score[h][s]))
    return total


def gamma_power(gamma: float, c: int) -> float:
    """gamma^c as the float32 product of c factors, left to right (returned
    as the exact float64 value of that float32)."""
    g = np.float32(gamma)
    r = np.float32(1.0)
    for _ in range(c):
        r = np.float32(r * g)
    return float(r)


def select_memory(candidates, slot_block, key_score, M: int, gamma: float) -> list[int]:
    """The kept slots, in pick order: min(M, len(candidates)) greedy picks.

    Each block offers its best remaining candidate (largest Q, ties to the
    smaller slot) with gain Q * gamma^c, c = picks from that block so far;
    the largest gain wins, ties to the smaller c, then the smaller slot."""
    score = {s: slot_score(key_score, s) for s in candidates}
    by_block: dict[int, list[int]] = {}
    for s in candidates:
        by_block.setdefault(int(slot_block[s]), []).append(s)
    for b in by_block:
        by_block[b].sort(key=lambda s: (-score[s], s))
    taken = {b: 0 for b in by_block}
    picks = []
    for _ in range(min(M, len(candidates))):
        best = None  # (gain, c, slot, block)
        for b, rest in by_block.items():
            if taken[b] == len(rest):
                continue
            s = rest[taken[b]]
            gain = score[s] * gamma_power(gamma, taken[b])
            key = (gain, -taken[b], -s)
            if best is None or key > best[0]:
                best = (key, s, b)
        picks.append(best[1])
        taken[best[2]] += 1
    return picks


def memory_objective(kept, slot_block, key_score, gamma: float) -> float:
    """sum over blocks of sum_k Q_(k) gamma^k for a kept set (exact float64
    evaluation of the objective the selection maximises)."""
    by_block: dict[int, list[float]] = {}
    for s in kept:
        by_block.setdefault(int(slot_block[s]), []).append(slot_score(key_score, s))
    total = 0.0
    for vals in by_block.values():
        for k, v in enumerate(sorted(vals, reverse=True)):
            total += v * gamma_power(gamma, k)
    return total
