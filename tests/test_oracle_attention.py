"""Pins for the oracle's block-causal chunk attention with the cache bias.

* Brute force: pure-Python loops with math.exp on the tiny workload
  (2 heads, d 64, 96 slots, 32 new tokens over the oldest block, bias -0.5).
* Library routine: with bias 0 the result equals torch's float64
  scaled_dot_product_attention under the same boolean mask.
* Closed forms: one visible key returns its V; V == 1 gives 1 (weights sum
  to one); Q = 0 gives (e^b sum_hist v + sum_cur v) / (e^b n_hist + n_cur),
  which pins both the bias and the visibility; a bias of -1e30 leaves only
  the query's own block.
* Invariants: permuting slots (with their positions and blocks) changes
  nothing; the rows of block b in a multi-block query equal a streaming call
  for block b alone; RoPE on both sides makes a position shift of queries
  and keys invisible.
* Per-query blocks and the same-block mask: an explicit block array equal
  to the (q_block0, q_block_len) formula gives the same result; blocks of
  unequal length (the first block one frame longer) follow the brute-force
  loop; the same-block mask equals, block by block, plain attention over
  only that block's slots (a different route: slicing, no mask).
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import chunk_attention, ring_attention
from oracle.ring import Ring
from oracle.rope import rope
from synthetic_inputs import WORKLOADS, normal_f32


def tiny_ring_and_queries():
    """The tiny workload: 3 history blocks of 32 at positions 0..95, then a
    block of 32 at positions 96..127 written over slots 0..31."""
    w = WORKLOADS["tiny"]
    rng = np.random.default_rng(w.seed)
    H, d, N, B = w.heads, w.head_dim, w.n_slots, w.extra["block_len"]
    ring = Ring(N, H, d, w.kv_dtype, w.rope_base)
    for b in range(4):
        _, k = normal_f32(rng, (B, H, d))
        _, v = normal_f32(rng, (B, H, d))
        ring.write(k, v, B, B * b, b)
        if b < 3:
            ring.advance(B)
    _, q = normal_f32(rng, (B, H, d))
    return ring, q, w


def brute_force(ring, q, q_pos0, q_block0, q_block_len, bias, sigma):
    K, V = ring.k_values(), ring.v_values()
    H, N, d = K.shape
    n_q = q.shape[0]
    out = np.zeros((n_q, H, d))
    lse = np.zeros((H, n_q))
    for i in range(n_q):
        pos = q_pos0 + i
        bq = q_block0 + i // q_block_len
        for h in range(H):
            qr = [0.0] * d
            for j in range(d // 2):
                phi = pos * ring.rope_base ** (-2.0 * j / d)
                c, s = math.cos(phi), math.sin(phi)
                x0, x1 = q[i, h, 2 * j], q[i, h, 2 * j + 1]
                qr[2 * j] = x0 * c - x1 * s
                qr[2 * j + 1] = x0 * s + x1 * c
            logits = {}
            for s_ in range(N):
                b = int(ring.slot_block[s_])
                if b == -1 or b > bq:
                    continue
                dot = sum(qr[t] * K[h, s_, t] for t in range(d))
                logits[s_] = sigma * dot + (bias if b < bq else 0.0)
            mx = max(logits.values())
            w = {s_: math.exp(l - mx) for s_, l in logits.items()}
            tot = sum(w.values())
            for t in range(d):
                out[i, h, t] = sum(w[s_] * V[h, s_, t] for s_ in w) / tot
            lse[h, i] = mx + math.log(tot)
    return out, lse


def test_bruteforce_tiny():
    ring, q, w = tiny_ring_and_queries()
    sigma = 1 / math.sqrt(w.head_dim)
    out, lse = ring_attention(ring, q, 96, 3, 32, w.cache_bias)
    # brute force row by row (each row at its own position)
    for r in (0, 5, 31):
        bo1, bl1 = brute_force(ring, q[r:r + 1], 96 + r, 3, 32, w.cache_bias, sigma)
        assert np.allclose(out[r], bo1[0], atol=1e-12, rtol=0)
        assert np.allclose(lse[:, r], bl1[:, 0], atol=1e-12, rtol=0)


def test_bias_zero_matches_torch_sdpa():
    ring, q, w = tiny_ring_and_queries()
    out, _ = ring_attention(ring, q, 96, 3, 32, 0.0)
    K = torch.from_numpy(ring.k_values())
    V = torch.from_numpy(ring.v_values())
    qr = torch.from_numpy(rope(q, (96 + np.arange(32))[:, None], w.rope_base))
    mask = torch.from_numpy((ring.slot_block != -1) & (ring.slot_block <= 3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qr.permute(1, 0, 2), K, V, attn_mask=mask[None, None, :].expand(w.heads, 32, -1))
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_single_visible_key_returns_v():
    rng = np.random.default_rng(11)
    H, d, N = 2, 64, 10
    K = rng.standard_normal((H, N, d))
    V = rng.standard_normal((H, N, d))
    blk = np.full(N, -1)
    blk[7] = 0
    q = rng.standard_normal((3, H, d)) * 10
    out, lse = chunk_attention(K, V, blk, q, 0, 0, 3, -2.0, 0.0, 10000.0)
    assert np.allclose(out, np.broadcast_to(V[:, 7, :][None], out.shape), atol=1e-14)


def test_rows_sum_to_one():
    ring, q, w = tiny_ring_and_queries()
    ones = np.ones_like(ring.v_values())
    out, _ = chunk_attention(ring.k_values(), ones, ring.slot_block, q * 7, 96, 3, 32,
                             w.cache_bias, 0.0, w.rope_base)
    assert np.allclose(out, 1.0, atol=1e-13)


@pytest.mark.parametrize("beta", [0.0, -0.5, -4.0, 0.3])
def test_zero_query_closed_form(beta):
    ring, q, w = tiny_ring_and_queries()
    out, lse = ring_attention(ring, np.zeros_like(q), 96, 3, 32, beta)
    V = ring.v_values()
    hist = ring.slot_block < 3
    cur = ring.slot_block == 3
    num = math.exp(beta) * V[:, hist].sum(1) + V[:, cur].sum(1)
    den = math.exp(beta) * hist.sum() + cur.sum()
    assert np.allclose(out, (num / den)[None], atol=1e-13)
    assert np.allclose(lse, math.log(den), atol=1e-13)


def test_large_negative_bias_leaves_current_block():
    ring, q, w = tiny_ring_and_queries()
    out, _ = ring_attention(ring, q, 96, 3, 32, -1e30)
    blk = ring.slot_block.copy()
    blk[blk < 3] = -1
    ref, _ = chunk_attention(ring.k_values(), ring.v_values(), blk, q, 96, 3, 32, 0.0, 0.0,
                             w.rope_base)
    assert np.allclose(out, ref, atol=1e-13)


def test_slot_permutation_invariance():
    ring, q, w = tiny_ring_and_queries()
    out, lse = ring_attention(ring, q, 96, 3, 32, w.cache_bias)
    perm = np.random.default_rng(2).permutation(ring.N)
    out2, lse2 = chunk_attention(ring.k_values()[:, perm], ring.v_values()[:, perm],
                                 ring.slot_block[perm], q, 96, 3, 32, w.cache_bias, 0.0,
                                 w.rope_base)
    assert np.allclose(out, out2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)


def test_streaming_block_equals_multiblock_rows():
    rng = np.random.default_rng(12)
    H, d, B, nb = 2, 64, 8, 4
    N = B * nb
    ring = Ring(N, H, d, "f32", 10000.0)
    qs = []
    for b in range(nb):
        _, k = normal_f32(rng, (B, H, d))
        _, v = normal_f32(rng, (B, H, d))
        _, qq = normal_f32(rng, (B, H, d))
        ring.write(k, v, B, B * b, b)
        ring.advance(B)
        qs.append(qq)
    q = np.concatenate(qs)
    full, full_lse = ring_attention(ring, q, 0, 0, B, -0.7)
    for b in range(nb):
        one, one_lse = ring_attention(ring, qs[b], B * b, b, B, -0.7)
        assert np.allclose(full[B * b:B * (b + 1)], one, atol=1e-13)
        assert np.allclose(full_lse[:, B * b:B * (b + 1)], one_lse, atol=1e-13)
    # block 0 sees only itself: equal to plain attention over its 8 keys
    blk = ring.slot_block.copy()
    blk[blk > 0] = -1
    ref, _ = chunk_attention(ring.k_values(), ring.v_values(), blk, qs[0], 0, 0, B, 5.0, 0.0,
                             10000.0)
    assert np.allclose(full[:B], ref, atol=1e-13)


def test_position_shift_invariance():
    # Rotating cached keys by delta and shifting the queries' positions by the
    # same delta leaves attention unchanged (relative positions only).
    ring, q, w = tiny_ring_and_queries()
    out, _ = ring_attention(ring, q, 96, 3, 32, w.cache_bias)
    Kr = rope(ring.k_values(), np.full((1, ring.N), -1000), w.rope_base)
    out2, _ = chunk_attention(Kr, ring.v_values(), ring.slot_block, q, 96 - 1000, 3, 32,
                              w.cache_bias, 0.0, w.rope_base)
    assert np.allclose(out, out2, atol=1e-10)


def test_no_visible_key_row():
    H, d, N = 1, 4, 6
    K = np.ones((H, N, d))
    V = np.ones((H, N, d))
    blk = np.array([5, 5, 5, -1, -1, -1])
    q = np.ones((2, H, d))
    out, lse = chunk_attention(K, V, blk, q, 0, 4, 1, 0.0, 0.0, 0.0)  # blocks 4, 5
    assert np.all(out[0] == 0) and lse[0, 0] == -np.inf
    assert np.allclose(out[1], 1.0) and np.isfinite(lse[0, 1])


def test_two_key_closed_form():
    # d = 2, no RoPE, sigma = 1: q = (1, 0); keys (1, 0) in an earlier block
    # and (0, 1) in the query's block; bias b on the first only.
    K = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    V = np.array([[[2.0, 0.0], [0.0, 3.0]]])
    blk = np.array([0, 1])
    q = np.array([[[1.0, 0.0]]])
    for b in (0.0, -0.5, 0.3):
        out, lse = chunk_attention(K, V, blk, q, 0, 1, 1, b, 1.0, 0.0)
        w0 = math.exp(1.0 + b) / (math.exp(1.0 + b) + 1.0)
        assert np.allclose(out[0, 0], [2 * w0, 3 * (1 - w0)], atol=1e-15)
        assert abs(lse[0, 0] - math.log(math.exp(1 + b) + 1)) < 1e-15


def test_query_block_array_equals_formula():
    ring, q, w = tiny_ring_and_queries()
    a = ring_attention(ring, q, 96, 2, 10, -0.5)
    qb = 2 + np.arange(q.shape[0]) // 10
    b = ring_attention(ring, q, 96, 0, 1, -0.5, q_blocks=qb)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_unequal_blocks_brute_force():
    """Queries in blocks of 12, 10 and 10 (a longer first block): each query
    row equals the brute-force loop run for that query alone."""
    ring, q, w = tiny_ring_and_queries()
    sizes = [12, 10, 10]
    qb = np.repeat([1, 2, 3], sizes)
    out, lse = ring_attention(ring, q, 96, 0, 1, -0.5, q_blocks=qb)
    sigma = 1 / math.sqrt(q.shape[2])
    for i in (0, 11, 12, 21, 22, 31):
        ref, ref_lse = brute_force(ring, q[i:i + 1], 96 + i, int(qb[i]), 1, -0.5, sigma)
        assert np.max(np.abs(out[i] - ref[0])) < 1e-12
        assert np.max(np.abs(lse[:, i] - ref_lse[:, 0])) < 1e-12


def test_same_block_mask_equals_sliced_plain_attention():
    """Text cross-attention: 3 segments' prompts (block ids 0, 1, 2; one slot
    empty), queries of segments 2, 0, 1.  Each query block's rows equal plain
    attention over only that segment's slots, with every slot relabelled
    into one visible block."""
    rng = np.random.default_rng(9)
    H, d, N = 2, 16, 40
    blk = np.array([0] * 12 + [1] * 9 + [2] * 18 + [-1])
    k = rng.standard_normal((H, N, d))
    v = rng.standard_normal((H, N, d))
    q = rng.standard_normal((15, H, d))
    qb = np.repeat([2, 0, 1], 5)
    out, lse = chunk_attention(k, v, blk, q, 0, 0, 1, -3.0, 0.0, 0.0, q_blocks=qb, mask="same")
    for seg in (0, 1, 2):
        rows, cols = qb == seg, blk == seg
        ref, ref_lse = chunk_attention(k[:, cols], v[:, cols], np.zeros(cols.sum(), np.int64), q[rows],
                                       0, 0, rows.sum(), -3.0, 0.0, 0.0)
        assert np.allclose(out[rows], ref, atol=1e-13) and np.allclose(lse[:, rows], ref_lse, atol=1e-13)
    # a segment with no text slots: zero output, lse -inf
    out2, lse2 = chunk_attention(k, v, blk, q[:3], 0, 0, 1, 0.0, 0.0, 0.0, q_blocks=[3, 3, 3], mask="same")
    assert np.all(out2 == 0) and np.all(lse2 == -np.inf)
