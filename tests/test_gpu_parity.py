"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case uses seeded synthetic N(0,1) inputs (synthetic_inputs.py) with the
workload shapes: the tiny case, one streaming layer (757 new over 5,788 fp8
slots, 40 heads, d 128), ring wrap + position reset, and joint audio-video
block-causal attention (bf16, 32 heads).  Bookkeeping and masks must be
bit-exact, FP8 codes within one step, attention within the tolerances in
gpu_helpers.ATTN_TOL.  Attention is compared with the oracle fed the GPU's
own cache contents (so write rounding is not counted twice) and, end to end,
with the oracle's own cache.
"""
import math
import sys

import numpy as np
import pytest
import torch

from autoregressive_video_diffusion_ring_amd import RcError, Ring
from oracle import e4m3
from oracle.attention import chunk_attention, ring_attention, visibility, query_blocks
from oracle.ring import Ring as OracleRing
from synthetic_inputs import WORKLOADS

from gpu_helpers import (DEV, assert_attention_close, compare_cache, gpu_cache, inputs, oracle_from_gpu,
                         oracle_rows, rel_l2, to_np64)

pytestmark = pytest.mark.gpu


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU", allow_module_level=True)


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def make_pair(N, H, d, kv, rope, first_slot=0, n_anchor=0):
    return (Ring(N, H, d, kv, rope, first_slot=first_slot, n_anchor=n_anchor, device=DEV),
            OracleRing(N, H, d, kv, rope, first_slot=first_slot, n_anchor=n_anchor))


def write_both(g, o, rng, n, pos0, blk):
    kt, k = inputs(rng, g.kv_name, (n, g.H, g.d))
    vt, v = inputs(rng, g.kv_name, (n, g.H, g.d))
    g.write(kt, vt, pos0, blk)
    o.write(k, v, n, pos0, blk)
    return kt, vt


# ------------------------------------------------------------------ tiny
def test_tiny_end_to_end():
    w = WORKLOADS["tiny"]
    banner("tiny: f32 ring N=96 H=2 d=64, 4 blocks of 32, bias -0.5")
    rng = np.random.default_rng(w.seed)
    B = w.extra["block_len"]
    g, o = make_pair(w.n_slots, w.heads, w.head_dim, w.kv_dtype, w.rope_base)
    for b in range(4):
        write_both(g, o, rng, B, B * b, b)
        if b < 3:
            g.advance(B)
            o.advance(B)
    qt, q = inputs(rng, "f32", (B, w.heads, w.head_dim))
    lse = torch.empty((w.heads, B), dtype=torch.float32, device=DEV)
    out = g.attention(qt, 96, 3, B, w.cache_bias, lse=lse)
    compare_cache(gpu_cache(g), o, "f32")
    ref_gpu, lse_gpu_ref = ring_attention(oracle_from_gpu(g, w.rope_base), q, 96, 3, B, w.cache_bias)
    assert_attention_close(out, ref_gpu, "f32")
    assert np.max(np.abs(to_np64(lse) - lse_gpu_ref)) < 1e-5
    ref, _ = ring_attention(o, q, 96, 3, B, w.cache_bias)
    assert_attention_close(out, ref, "f32")


# ------------------------------------------------------------------ writes
def permute_slots(g, perm):
    """Move every slot of an FP8 ring (K row, V^T column, scales, position,
    block) to the physical slot perm[s] was at: slot s gets old slot perm[s]."""
    H, N, d = g.H, g.N, g.d
    p = torch.from_numpy(np.asarray(perm)).to(DEV)
    kb = g.buffers[0].view(H, g.v_ld, d)[:, :N]
    kb.copy_(kb[:, p].clone())
    vb = g.buffers[1].view(H, d, g.v_ld)
    vb[:, :, :N] = vb[:, :, :N][:, :, p].clone()
    for i in (2, 3):
        sb = g.buffers[i].view(torch.float32)[:H * g.v_ld].view(H, g.v_ld)[:, :N]
        sb.copy_(sb[:, p].clone())
    for i in (4, 5):
        mb = g.buffers[i].view(torch.int32)[:N]
        mb.copy_(mb[p].clone())
    torch.cuda.synchronize()


def stream_ring(seed, head0=0, H=40, d=128, N=5788, n_hist=5031, n_new=757):
    """History of n_hist tokens (block 0, positions 0..n_hist-1) committed,
    then the current chunk of n_new tokens (block 1) written."""
    rng = np.random.default_rng(seed)
    g, o = make_pair(N, H, d, "fp8", 10000.0, first_slot=head0)
    write_both(g, o, rng, n_hist, 0, 0)
    g.advance(n_hist)
    o.advance(n_hist)
    write_both(g, o, rng, n_new, n_hist, 1)
    return g, o, rng


def test_write_stream_full_size():
    banner("write: fp8 N=5788 H=40 d=128, 5031 history + 757 current")
    g, o, _ = stream_ring(WORKLOADS["stream"].seed)
    compare_cache(gpu_cache(g), o, "fp8")


@pytest.mark.parametrize("head0", [4000, 5400])
def test_write_wrap_and_rewrite(head0):
    banner(f"write: wrap at head {head0}, then a second pass over the same chunk")
    rng = np.random.default_rng(WORKLOADS["wrap"].seed)
    N, H, d = 5788, 40, 128
    g, o = make_pair(N, H, d, "fp8", 10000.0, first_slot=head0)
    write_both(g, o, rng, 757, 5031, 1)
    compare_cache(gpu_cache(g), o, "fp8")
    # second denoising pass: new values, same slots, same state
    write_both(g, o, rng, 757, 5031, 1)
    c = gpu_cache(g)
    compare_cache(c, o, "fp8")
    slots = (head0 + np.arange(757)) % N
    assert set(np.nonzero(c["slot_block"] == 1)[0]) == set(slots)
    with pytest.raises(RcError):
        g.write(*(inputs(rng, "fp8", (757, H, d))[0] for _ in range(2)), 5032, 1)
    assert g.state() == o.state()


@pytest.mark.parametrize("kv,d,H,head0", [("fp8", 128, 40, 1234), ("bf16", 64, 8, 5787)])
def test_write_whole_ring_one_call(kv, d, H, head0):
    """The largest write: n_new = N tokens in one call from a head inside the
    ring, so the write wraps and every slot is overwritten; then attention of
    the chunk's last 96 queries over all N slots (one block, all visible)."""
    banner(f"write: whole ring in one call, {kv} d={d} N=5788 H={H} from head {head0}; attention over it")
    rng = np.random.default_rng(WORKLOADS["wrap"].seed + 11)
    N = 5788
    g, o = make_pair(N, H, d, kv, 10000.0, first_slot=head0)
    write_both(g, o, rng, N, 2000, 0)
    c = gpu_cache(g)
    compare_cache(c, o, kv)
    assert (c["slot_block"] == 0).all()
    assert np.array_equal(c["slot_pos"][(head0 + np.arange(N)) % N], 2000 + np.arange(N))
    qt, q = inputs(rng, kv, (96, H, d))
    out = g.attention(qt, 2000 + N - 96, 0, 96, -0.5)
    ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, 2000 + N - 96, 0, 96, -0.5)
    assert_attention_close(out, ref, kv)
    g.advance(N)
    o.advance(N)
    assert g.state() == o.state()


@pytest.mark.parametrize("kv,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("fp8", 64)])
def test_write_other_formats(kv, d):
    banner(f"write: {kv} d={d} ragged chunks with wrap")
    rng = np.random.default_rng(11)
    N, H = 200, 3
    g, o = make_pair(N, H, d, kv, 10000.0, first_slot=170)
    write_both(g, o, rng, 77, 1000, 0)
    g.advance(77)
    o.advance(77)
    write_both(g, o, rng, 150, 1077, 1)
    compare_cache(gpu_cache(g), o, kv)


@pytest.mark.parametrize("kv,d", [("fp8", 128), ("fp8", 64), ("bf16", 128), ("f32", 64)])
def test_write_single_tokens(kv, d):
    """One-token writes: a chunk of one slot inside a 32-slot group, at the
    ring's last slot, then at slot 0 after the wrap, with two passes over the
    same token; each compared with the oracle, neighbours untouched."""
    banner(f"write: {kv} d={d} single tokens at slots 37, 199, 0 (N=200, H=3)")
    rng = np.random.default_rng(12)
    N, H = 200, 3
    g, o = make_pair(N, H, d, kv, 10000.0, first_slot=37)
    write_both(g, o, rng, 1, 5, 0)
    compare_cache(gpu_cache(g), o, kv)
    g.advance(1)
    o.advance(1)
    # move the head to the last slot with a 161-token chunk, then one token there
    write_both(g, o, rng, 161, 6, 1)
    g.advance(161)
    o.advance(161)
    assert g.state()[0] == 199
    for blk, pos in ((2, 167), (3, 168)):
        for _ in range(2):  # two denoising passes over the same token
            write_both(g, o, rng, 1, pos, blk)
            compare_cache(gpu_cache(g), o, kv)
        g.advance(1)
        o.advance(1)
    c = gpu_cache(g)
    assert c["slot_block"][199] == 2 and c["slot_block"][0] == 3 and c["slot_block"][1] == -1
    assert g.state() == o.state()


@pytest.mark.parametrize("kv,d,N,A,n,H,chunks", [
    ("fp8", 128, 300, 50, 77, 3, 9),       # chunk 0 straddles the anchor; ragged wraps to slot 50
    ("bf16", 64, 200, 64, 40, 3, 10),
    ("fp8", 128, 5788, 757, 757, 8, 9),    # the streaming shape with the first chunk pinned
])
def test_anchor_ring_stream(kv, d, N, A, n, H, chunks):
    """Anchor + sliding window: the first A tokens stay pinned in slots 0..A-1
    while the ring part A..N-1 wraps.  Cache contents and bookkeeping after
    every write (and a second pass over a wrapping chunk), then a position
    reset, then block-causal attention over the whole cache."""
    banner(f"anchor ring: {kv} d={d} N={N} A={A} chunks of {n}, H={H}, {chunks} chunks")
    rng = np.random.default_rng(41)
    g, o = make_pair(N, H, d, kv, 10000.0, n_anchor=A)
    wrapped = False
    for b in range(chunks):
        write_both(g, o, rng, n, n * b, b)
        compare_cache(gpu_cache(g), o, kv)
        if g.state()[0] + n > N:   # this chunk wraps: a second pass must hit the same slots
            wrapped = True
            write_both(g, o, rng, n, n * b, b)
            compare_cache(gpu_cache(g), o, kv)
        if b + 1 < chunks:
            g.advance(n)
            o.advance(n)
    assert wrapped
    c = gpu_cache(g)   # the anchor still holds the first A tokens of the stream
    assert np.array_equal(c["slot_pos"][:A], np.arange(A))
    assert np.array_equal(c["slot_block"][:A], np.arange(A) // n)
    g.rerotate(-1000)
    o.rerotate(-1000)
    c = gpu_cache(g)
    assert np.array_equal(c["slot_pos"][:A], np.arange(A) - 1000)
    q_pos0, q_blk = n * (chunks - 1) - 1000, chunks - 1
    qt, q = inputs(rng, kv, (n, H, d))
    out = g.attention(qt, q_pos0, q_blk, n, -0.5)
    rows = np.r_[0:n:max(1, n // 60), n - 3:n]
    ref, _ = oracle_rows(oracle_from_gpu(g, 10000.0), q, rows, q_pos0, q_blk, n, -0.5)
    assert_attention_close(out, ref, kv, rows=rows)


# ------------------------------------------------------------------ rerotate
@pytest.mark.parametrize("kv,d", [("fp8", 128), ("bf16", 64), ("f32", 64)])
def test_rerotate_zero_large_and_partial(kv, d):
    """Degenerate and extreme shifts on a partly filled, wrapped ring (300
    slots, 130 written from slot 250): delta 0 (the identity rotation, up to
    requantisation), then +200,000 positions; every occupied slot matches the
    oracle, and the 170 empty slots keep their bytes and positions."""
    banner(f"rerotate: {kv} d={d} N=300 H=3, 130 of 300 slots written from slot 250; delta 0 then +200000")
    rng = np.random.default_rng(33)
    N, H = 300, 3
    g, o = make_pair(N, H, d, kv, 10000.0, first_slot=250)
    write_both(g, o, rng, 130, 70, 4)
    g.advance(130)
    o.advance(130)
    c0 = gpu_cache(g)
    empty = c0["slot_block"] == -1
    assert int(empty.sum()) == 170
    for delta in (0, 200_000):
        ref = oracle_from_gpu(g, 10000.0)
        g.rerotate(delta)
        ref.rerotate(delta)
        o.rerotate(delta)
        c = gpu_cache(g)
        compare_cache(c, ref, kv)
        assert c["state"] == o.state()
        assert np.array_equal(c["k"][:, empty], c0["k"][:, empty])
        assert np.array_equal(c["slot_pos"][empty], c0["slot_pos"][empty])
        if kv == "fp8":
            assert np.array_equal(c["k_scale"][:, empty], c0["k_scale"][:, empty])
    # positions moved by the sum of the shifts
    assert np.array_equal(c["slot_pos"][~empty], c0["slot_pos"][~empty] + 200_000)
    # V is never touched by a re-rotation
    assert np.array_equal(c["v"], c0["v"])


def test_rerotate_wrap_reset():
    banner("rerotate: head 5400 (wrapped current chunk), delta -3000 over all slots")
    head0 = (5400 - 5031) % 5788
    g, o, rng = stream_ring(WORKLOADS["wrap"].seed, head0=head0)
    # the current chunk starts at slot 5400 and wraps
    assert g.state()[0] == 5400
    before = oracle_from_gpu(g, 10000.0)
    g.rerotate(-3000)
    before.rerotate(-3000)
    compare_cache(gpu_cache(g), before, "fp8")
    # against re-encoding from scratch: dequantised keys within two steps
    o.rerotate(-3000)
    fresh = OracleRing(5788, 40, 128, "fp8", 10000.0, first_slot=head0)
    rng2 = np.random.default_rng(WORKLOADS["wrap"].seed)
    from gpu_helpers import inputs as _inp  # same draws as stream_ring
    _, k0 = _inp(rng2, "fp8", (5031, 40, 128))
    _, v0 = _inp(rng2, "fp8", (5031, 40, 128))
    fresh.write(k0, v0, 5031, -3000, 0)
    fresh.advance(5031)
    _, k1 = _inp(rng2, "fp8", (757, 40, 128))
    _, v1 = _inp(rng2, "fp8", (757, 40, 128))
    fresh.write(k1, v1, 757, 5031 - 3000, 1)
    gk = oracle_from_gpu(g, 10000.0).k_values()
    s = np.maximum(fresh.k_scale, gpu_cache(g)["k_scale"]).astype(np.float64)[..., None]
    assert np.all(np.abs(gk - fresh.k_values()) <= 3 * 16 * math.sqrt(2) * s)
    assert g.state() == fresh.state()


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("kv,d", [("fp8", 128), ("fp8", 64), ("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_attention_ragged_multiblock(kv, d):
    """Several tiles and a ragged tail on both axes, a wrapped ring with empty
    slots, multi-block queries (block-causal) and a nonzero bias."""
    banner(f"attention: {kv} d={d} N=300 H=3, 150 queries in 3 blocks, bias -0.5")
    rng = np.random.default_rng(21)
    N, H = 300, 3
    g, o = make_pair(N, H, d, kv, 10000.0, first_slot=250)
    for b, (n, p0) in enumerate([(60, 1000), (70, 1060), (50, 1130)]):
        write_both(g, o, rng, n, p0, b)
        g.advance(n)
        o.advance(n)
    # queries: blocks 1..3, 50 each; block 3 has no keys of its own
    qt, q = inputs(rng, kv, (150, H, d))
    lse = torch.empty((H, 150), dtype=torch.float32, device=DEV)
    out = g.attention(qt, 1060, 1, 50, -0.5, lse=lse)
    ref, ref_lse = ring_attention(oracle_from_gpu(g, 10000.0), q, 1060, 1, 50, -0.5)
    assert_attention_close(out, ref, kv)
    lse_tol = {"fp8": 5e-2, "bf16": 2e-2, "f32": 1e-5}[kv]
    assert np.max(np.abs(to_np64(lse) - ref_lse)) < lse_tol
    ref2, _ = ring_attention(o, q, 1060, 1, 50, -0.5)
    assert_attention_close(out, ref2, kv)


@pytest.mark.parametrize("kv,d", [("fp8", 128), ("bf16", 64), ("f32", 64)])
def test_attention_single_query_and_softmax_scale(kv, d):
    """One query (the smallest call), then 70 queries in two blocks with
    softmax scales other than 1/sqrt(d) (0.05 and 0.5), over a wrapped ring
    of three blocks with a bias on the earlier ones."""
    banner(f"attention: {kv} d={d} N=200 H=2, one query; then softmax scale 0.05 and 0.5")
    rng = np.random.default_rng(44)
    N, H = 200, 2
    g, o = make_pair(N, H, d, kv, 10000.0, first_slot=170)
    for b, (n, p0) in enumerate([(64, 500), (64, 564), (40, 628)]):
        write_both(g, o, rng, n, p0, b)
        g.advance(n)
        o.advance(n)
    qt, q = inputs(rng, kv, (1, H, d))
    out = g.attention(qt, 667, 2, 1, -0.3)
    ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, 667, 2, 1, -0.3)
    assert_attention_close(out, ref, kv)
    qt, q = inputs(rng, kv, (70, H, d))
    for scale in (0.05, 0.5):
        out = g.attention(qt, 600, 1, 35, -0.3, scale)
        ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, 600, 1, 35, -0.3, scale)
        assert_attention_close(out, ref, kv)
        ref2, _ = ring_attention(o, q, 600, 1, 35, -0.3, scale)
        assert_attention_close(out, ref2, kv)


def test_attention_zero_rows_and_scale_spread():
    """Degenerate and extreme rows: all-zero K rows (scale 0), all-zero V rows
    (scale 0: the row still carries its softmax weight, so the sum must count
    it), and V rows scaled by 2^10 and 2^-10 so that per-slot V scales span
    2^20.  Powers of two keep the bf16 inputs exact."""
    banner("attention: fp8 with zero K / V rows and V scales spread over 2^20")
    rng = np.random.default_rng(33)
    N, H, d = 320, 4, 128
    g, o = make_pair(N, H, d, "fp8", 10000.0)
    for b, (n, p0) in enumerate([(120, 0), (110, 120), (80, 230)]):
        kt, k = inputs(rng, "fp8", (n, H, d))
        vt, v = inputs(rng, "fp8", (n, H, d))
        pick = rng.integers(0, 6, size=(n, H))
        for sel, kind in ((pick == 0, "k0"), (pick == 1, "v0"), (pick == 2, "vbig"), (pick == 3, "vsmall")):
            m = torch.from_numpy(sel).to(DEV)
            if kind == "k0":
                kt[m] = 0
                k[sel] = 0.0
            elif kind == "v0":
                vt[m] = 0
                v[sel] = 0.0
            else:
                f = 1024.0 if kind == "vbig" else 1.0 / 1024.0
                vt[m] = vt[m] * f
                v[sel] = v[sel] * f
        g.write(kt, vt, p0, b)
        o.write(k, v, n, p0, b)
        g.advance(n)
        o.advance(n)
    qt, q = inputs(rng, "fp8", (80, H, d))
    out = g.attention(qt, 230, 2, 80, -0.5)
    ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, 230, 2, 80, -0.5)
    # Attention is linear in V: with V rows carrying factors up to 2^10 the
    # outputs are up to 2^10 times those of unit-variance inputs, and so is
    # the error; the unit-variance bound applies to out / 2^10.
    assert_attention_close(to_np64(out) / 1024.0, ref / 1024.0, "fp8")
    ref2, _ = ring_attention(o, q, 230, 2, 80, -0.5)
    assert_attention_close(to_np64(out) / 1024.0, ref2 / 1024.0, "fp8")


def test_attention_stream_full_size_all_rows():
    """The streaming layer at its stated size, every one of the 757 rows,
    against both oracles: the oracle over the GPU's cache codes (the
    attention alone) and the oracle's own write chain (write + attention end
    to end)."""
    banner("attention: streaming layer 757 x 5788 fp8, 40 heads, all rows vs both oracles")
    g, o, rng = stream_ring(WORKLOADS["stream"].seed)
    qt, q = inputs(rng, "fp8", (757, 40, 128))
    lse = torch.empty((40, 757), dtype=torch.float32, device=DEV)
    out = g.attention(qt, 5031, 1, 757, 0.0, lse=lse)
    ref, ref_lse = ring_attention(oracle_from_gpu(g, 10000.0), q, 5031, 1, 757, 0.0)
    err, r = assert_attention_close(out, ref, "fp8")
    print(f"  vs oracle over GPU codes: max-abs {err:.3e}, rel-L2 {r:.3e}", flush=True)
    assert np.max(np.abs(to_np64(lse) - ref_lse)) < 5e-2
    ref2, _ = ring_attention(o, q, 5031, 1, 757, 0.0)
    err, r = assert_attention_close(out, ref2, "fp8")
    print(f"  vs oracle write chain:    max-abs {err:.3e}, rel-L2 {r:.3e}", flush=True)
    # determinism: the same call twice gives identical bits
    out2 = g.attention(qt, 5031, 1, 757, 0.0)
    assert torch.equal(out, out2)


def test_reset_full_size():
    """Ring wrap + position reset at its stated size: head at slot 5400 (the
    current chunk wraps), rerotate(-3000), then attention of the chunk's
    queries at their rebased positions.  Every row against the oracle over
    the GPU's codes and against the oracle's own write + rerotate chain, and
    against the same call before the reset."""
    banner("attention: 757 x 5788 x 40, head 5400, rerotate(-3000), rebased queries, all rows")
    head0 = (5400 - 5031) % 5788
    g, o, rng = stream_ring(WORKLOADS["wrap"].seed, head0=head0)
    assert g.state()[0] == 5400
    qt, q = inputs(rng, "fp8", (757, 40, 128))
    before = to_np64(g.attention(qt, 5031, 1, 757, -0.5))
    g.rerotate(-3000)
    o.rerotate(-3000)
    after = to_np64(g.attention(qt, 5031 - 3000, 1, 757, -0.5))
    ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, 5031 - 3000, 1, 757, -0.5)
    err, r = assert_attention_close(after, ref, "fp8")
    print(f"  vs oracle over GPU codes: max-abs {err:.3e}, rel-L2 {r:.3e}", flush=True)
    ref2, _ = ring_attention(o, q, 5031 - 3000, 1, 757, -0.5)
    err, r = assert_attention_close(after, ref2, "fp8")
    print(f"  vs oracle write chain:    max-abs {err:.3e}, rel-L2 {r:.3e}", flush=True)
    # RoPE: only relative positions matter, so the reset changes nothing beyond
    # the keys' FP8 re-quantisation
    assert_attention_close(after, before, "fp8")


def test_slot_permutation_full_size():
    """Moving slots (with their positions, blocks and scales) to a random
    permutation of the 5,788 physical slots changes nothing: every row
    against the oracle of the unpermuted ring, 757 x 5788 x 40."""
    banner("attention: 757 x 5788 x 40 after a random permutation of the physical slots")
    g, o, rng = stream_ring(WORKLOADS["stream"].seed + 11)
    qt, q = inputs(rng, "fp8", (757, 40, 128))
    ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, 5031, 1, 757, -0.5)
    a = to_np64(g.attention(qt, 5031, 1, 757, -0.5))
    permute_slots(g, np.random.default_rng(5).permutation(5788))
    b = to_np64(g.attention(qt, 5031, 1, 757, -0.5))
    err, r = assert_attention_close(b, ref, "fp8")
    print(f"  permuted vs oracle: max-abs {err:.3e}, rel-L2 {r:.3e}", flush=True)
    assert_attention_close(a, ref, "fp8")
    assert rel_l2(b, a) < 6e-2


def test_attention_query_magnitude_spread():
    """Queries whose magnitudes spread over 2^-6 .. 2^6 per (token, head),
    with the softmax scale taken 2^-6 lower so that the largest keep
    unit-variance logits.  Every row against the oracle; and each query's
    result depends on its own query only (one FP8 scale per query and head):
    zeroing the other queries of the call leaves its output bit-identical,
    in both operand precisions."""
    from autoregressive_video_diffusion_ring_amd import (RC_PRECISION_AUTO, RC_PRECISION_ONE_TERM,
                                                         RC_PRECISION_TWO_TERM, rc_set_attention_precision)
    banner("attention: query magnitudes spread 2^-6 .. 2^6 per (token, head), 256 x 5788 x 8")
    rng = np.random.default_rng(WORKLOADS["stream"].seed + 29)
    N, H, d, n_q = 5788, 8, 128, 256
    g, o = make_pair(N, H, d, "fp8", 10000.0)
    write_both(g, o, rng, 5031, 0, 0)
    g.advance(5031)
    o.advance(5031)
    write_both(g, o, rng, 757, 5031, 1)
    u = rng.integers(-6, 7, size=(n_q, H))
    _, q = inputs(rng, "fp8", (n_q, H, d))
    q = q * np.exp2(u)[..., None]  # exact in bfloat16 (power-of-two scaling)
    qt = torch.from_numpy(q.astype(np.float32)).to(DEV).to(torch.bfloat16)
    assert np.array_equal(to_np64(qt), q)
    sigma = 2.0 ** -6 / math.sqrt(d)
    orc = oracle_from_gpu(g, 10000.0)
    ref, _ = ring_attention(orc, q, 5031, 1, n_q, 0.0, sigma)
    keep = np.abs(u) < 3
    q_kept = torch.from_numpy(np.where(keep[..., None], q, 0.0).astype(np.float32)).to(DEV).to(torch.bfloat16)
    try:
        for mode in (RC_PRECISION_AUTO, RC_PRECISION_ONE_TERM, RC_PRECISION_TWO_TERM):
            rc_set_attention_precision(mode)
            out = g.attention(qt, 5031, 1, n_q, 0.0, softmax_scale=sigma)
            err, r = assert_attention_close(out, ref, "fp8")
            print(f"  precision mode {mode}: max-abs {err:.3e}, rel-L2 {r:.3e}", flush=True)
            out_kept = g.attention(q_kept, 5031, 1, n_q, 0.0, softmax_scale=sigma)
            same = (out.view(torch.int16) == out_kept.view(torch.int16)).all(dim=2).cpu().numpy()
            assert same[keep].all(), f"{(~same[keep]).sum()} (query, head) outputs changed"
    finally:
        rc_set_attention_precision(RC_PRECISION_AUTO)


def test_attention_after_reset_matches_before():
    """RoPE makes attention depend on relative positions only: after a reset
    by delta, queries moved by the same delta give the same result (within
    the FP8 re-quantisation of the keys)."""
    banner("attention: before vs after rerotate(-3000) with rebased queries")
    g, o, rng = stream_ring(7, H=8, N=1000, n_hist=700, n_new=200)
    qt, q = inputs(rng, "fp8", (200, 8, 128))
    a = to_np64(g.attention(qt, 700, 1, 200, -0.5))
    g.rerotate(-3000)
    b = to_np64(g.attention(qt, 700 - 3000, 1, 200, -0.5))
    assert_attention_close(b, a, "fp8")
    ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, -2300, 1, 200, -0.5)
    assert_attention_close(b, ref, "fp8")


def test_zero_query_closed_form():
    banner("attention: Q = 0 closed form (pins bias and visibility)")
    g, o, rng = stream_ring(8, H=4, N=700, n_hist=500, n_new=150)
    beta = -0.7
    q = torch.zeros((150, 4, 128), dtype=torch.bfloat16, device=DEV)
    out = to_np64(g.attention(q, 500, 1, 150, beta))
    orc = oracle_from_gpu(g, 10000.0)
    V = orc.v_values()
    hist, cur = orc.slot_block == 0, orc.slot_block == 1
    num = math.exp(beta) * V[:, hist].sum(1) + V[:, cur].sum(1)
    den = math.exp(beta) * hist.sum() + cur.sum()
    closed = np.broadcast_to((num / den)[None], out.shape)
    assert_attention_close(out, closed, "fp8")


def test_slot_permutation_invariance():
    banner("attention: permuting physical slots (with positions and blocks) changes nothing")
    g, o, rng = stream_ring(9, H=4, N=640, n_hist=500, n_new=100)
    qt, q = inputs(rng, "fp8", (100, 4, 128))
    a = to_np64(g.attention(qt, 500, 1, 100, -0.5))
    permute_slots(g, np.random.default_rng(2).permutation(640))
    b = to_np64(g.attention(qt, 500, 1, 100, -0.5))
    ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, 500, 1, 100, -0.5)
    assert_attention_close(a, ref, "fp8")
    assert_attention_close(b, ref, "fp8")
    # two independent FP8 roundings of P (different tile compositions)
    assert rel_l2(b, a) < 6e-2


def test_rows_without_visible_keys():
    banner("attention: queries of a block before every cached block")
    rng = np.random.default_rng(5)
    g, o = make_pair(128, 2, 128, "bf16", 0.0)
    write_both(g, o, rng, 100, 0, 5)
    qt, _ = inputs(rng, "bf16", (40, 2, 128))
    lse = torch.empty((2, 40), dtype=torch.float32, device=DEV)
    out = g.attention(qt, 0, 3, 20, 0.0, lse=lse)  # blocks 3 and 4: nothing visible
    assert torch.count_nonzero(out) == 0
    assert torch.all(torch.isneginf(lse))


# ------------------------------------------------------------------ joint A/V
def av_rings(seed):
    w = WORKLOADS["av"]
    rng = np.random.default_rng(seed)
    H, d, B = w.heads, w.head_dim, w.extra["blocks"]
    vb, ab = w.extra["video_block"], w.extra["audio_block"]
    gv, ov = make_pair(vb * B, H, d, "bf16", 0.0)
    ga, oa = make_pair(ab * B, H, d, "bf16", 0.0)
    for b in range(B):
        write_both(gv, ov, rng, vb, vb * b, b)
        write_both(ga, oa, rng, ab, ab * b, b)
        if b < B - 1:
            for r in (gv, ov, ga, oa):
                r.advance(vb if r in (gv, ov) else ab)
    qv = inputs(rng, "bf16", (vb * B, H, d))
    qa = inputs(rng, "bf16", (ab * B, H, d))
    return (gv, ov, ga, oa, qv, qa, vb, ab, B)


def test_joint_av_four_paths():
    banner("joint A/V: v->v, a->a, v->a, a->v, streaming block 9 and all 10 blocks, bf16 H=32")
    gv, ov, ga, oa, qv, qa, vb, ab, B = av_rings(WORKLOADS["av"].seed)
    ov_g, oa_g = oracle_from_gpu(gv, 0.0), oracle_from_gpu(ga, 0.0)
    for name, gring, oring, (qt, q), blen in [
        ("v->v", gv, ov_g, qv, vb), ("a->a", ga, oa_g, qa, ab),
        ("v->a", ga, oa_g, qv, vb), ("a->v", gv, ov_g, qa, ab)]:
        # streaming: the last block's queries only
        n = blen
        out = gring.attention(qt[(B - 1) * n:].contiguous(), 0, B - 1, n, 0.0)
        rows = np.unique(np.r_[0:n:max(1, n // 24), n - 1])
        qlast = q[(B - 1) * n:]
        ref, _ = oracle_rows(oring, qlast, rows, 0, B - 1, n, 0.0)
        assert_attention_close(out, ref, "bf16", rows=rows)
        # all blocks as queries (block-causal across them)
        out_all = gring.attention(qt, 0, 0, blen, 0.0)
        rows_all = np.unique(np.r_[0:B * blen:max(1, B * blen // 60), B * blen - 1])
        ref_all, _ = oracle_rows(oring, q, rows_all, 0, 0, blen, 0.0)
        assert_attention_close(out_all, ref_all, "bf16", rows=rows_all)
        print(f"  {name}: ok", flush=True)


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_per_query_blocks(d):
    """rc_chunk_attention_ex on an FP8 ring with RoPE: unequal blocks (100,
    170, 130, 140 tokens, so 32-query waves straddle block edges), every
    token's query carrying its block id; the block-causal mask with bias -0.4
    on earlier blocks, and the same-block mask.  All rows against the oracle
    over the GPU's own cache."""
    banner(f"fp8 d={d}: per-query blocks 100/170/130/140, both masks, bias -0.4")
    rng = np.random.default_rng(57)
    lens = [100, 170, 130, 140]
    N, H = 600, 2
    g, o = make_pair(N, H, d, "fp8", 10000.0)
    pos = 0
    for b, n in enumerate(lens):
        write_both(g, o, rng, n, pos, b)
        if b < len(lens) - 1:
            g.advance(n)
            o.advance(n)
        pos += n
    n_q = sum(lens)
    qt, q = inputs(rng, "fp8", (n_q, H, d))
    ids = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
    orc = oracle_from_gpu(g, 10000.0)
    for same in (False, True):
        out = g.attention(qt, 0, 0, None, -0.4, q_block=torch.from_numpy(ids).to(DEV), same_block=same)
        ref, _ = ring_attention(orc, q, 0, 0, 1, -0.4, q_blocks=ids, mask="same" if same else "causal")
        assert_attention_close(out, ref, "fp8")
        print(f"  {'same-block' if same else 'block-causal'}: ok", flush=True)


def test_joint_av_six_paths_first_block():
    """All six paths of the joint block with the first block one frame
    longer (1,536 video / 26 audio tokens, then 1,152 / 25) and three prompt
    segments: the four cache paths with per-query blocks (all ten blocks as
    queries, block-causal), and video->text, audio->text with the same-block
    mask (each block sees only its own segment's prompt)."""
    w = WORKLOADS["av6"]
    banner("joint A/V six paths: first block 1536/26, 3 prompt segments, bf16 H=32")
    rng = np.random.default_rng(w.seed)
    H, d, B = w.heads, w.head_dim, w.extra["blocks"]
    vlen = [w.extra["video_first"]] + [w.extra["video_block"]] * (B - 1)
    alen = [w.extra["audio_first"]] + [w.extra["audio_block"]] * (B - 1)
    seg, plen = w.extra["segment_of_block"], w.extra["prompt_tokens"]
    gv, ov = make_pair(sum(vlen), H, d, "bf16", 0.0)
    ga, oa = make_pair(sum(alen), H, d, "bf16", 0.0)
    gt, ot = make_pair(sum(plen), H, d, "bf16", 0.0)
    for b in range(B):
        write_both(gv, ov, rng, vlen[b], sum(vlen[:b]), b)
        write_both(ga, oa, rng, alen[b], sum(alen[:b]), b)
        for g_, o_, n_ in ((gv, ov, vlen[b]), (ga, oa, alen[b])):
            if b < B - 1:
                g_.advance(n_)
                o_.advance(n_)
    for sgm, n in enumerate(plen):   # each prompt's tokens carry their segment id as block id
        write_both(gt, ot, rng, n, 0, sgm)
        if sgm < len(plen) - 1:
            gt.advance(n)
            ot.advance(n)
    qv_t, qv = inputs(rng, "bf16", (sum(vlen), H, d))
    qa_t, qa = inputs(rng, "bf16", (sum(alen), H, d))
    vblk = np.repeat(np.arange(B), vlen).astype(np.int32)
    ablk = np.repeat(np.arange(B), alen).astype(np.int32)
    vseg = np.asarray(seg, dtype=np.int32)[vblk]
    aseg = np.asarray(seg, dtype=np.int32)[ablk]
    rings = {"v": (gv, oracle_from_gpu(gv, 0.0)), "a": (ga, oracle_from_gpu(ga, 0.0)),
             "t": (gt, oracle_from_gpu(gt, 0.0))}
    queries = {"v": (qv_t, qv, vblk, vseg), "a": (qa_t, qa, ablk, aseg)}
    for qn, kn in (("v", "v"), ("a", "a"), ("v", "a"), ("a", "v"), ("v", "t"), ("a", "t")):
        gring, oring = rings[kn]
        qt, q, qblk, qseg = queries[qn]
        same = kn == "t"
        ids = qseg if same else qblk
        out = gring.attention(qt, 0, 0, None, -0.4, q_block=torch.from_numpy(ids).to(DEV), same_block=same)
        n = q.shape[0]
        rows = np.unique(np.r_[0:n:max(1, n // 50), n - 1, 1535 if qn == "v" else 25, 1536 if qn == "v" else 26])
        rows = rows[rows < n]
        ref, _ = chunk_attention(oring.k_values(), oring.v_values(), oring.slot_block, q[rows], 0, 0, 1, -0.4, 0.0,
                                 0.0, q_blocks=ids[rows], mask="same" if same else "causal")
        assert_attention_close(out, ref, "bf16", rows=rows)
        print(f"  {qn}->{kn}: ok", flush=True)
    # streaming: the last block of video against its own segment's prompt
    last = vblk == B - 1
    out = gt.attention(qv_t[torch.from_numpy(last).to(DEV)].contiguous(), 0, seg[B - 1], int(last.sum()), 0.0,
                       same_block=True)
    sl = ot.slot_block == seg[B - 1]
    ref, _ = chunk_attention(ot.k_values()[:, sl], ot.v_values()[:, sl], np.zeros(sl.sum(), np.int64), qv[last],
                             0, 0, int(last.sum()), 0.0, 0.0, 0.0)
    assert_attention_close(out, ref, "bf16")


def test_split_kv_matches_unsplit():
    banner("attention: 25 audio queries over the 11520-slot video ring (split key range)")
    gv, ov, ga, oa, qv, qa, vb, ab, B = av_rings(4)
    qt, q = qa
    qlast = qt[(B - 1) * ab:].contiguous()
    assert gv.workspace_bytes(ab) > 0
    lse1 = torch.empty((32, ab), dtype=torch.float32, device=DEV)
    lse2 = torch.empty((32, ab), dtype=torch.float32, device=DEV)
    split = gv.attention(qlast, 0, B - 1, ab, -0.3, lse=lse1)
    nosplit = gv.attention(qlast, 0, B - 1, ab, -0.3, lse=lse2,
                           workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    ref, ref_lse = ring_attention(oracle_from_gpu(gv, 0.0), q[(B - 1) * ab:], 0, B - 1, ab, -0.3)
    assert_attention_close(split, ref, "bf16")
    assert_attention_close(nosplit, ref, "bf16")
    assert np.max(np.abs(to_np64(lse1) - ref_lse)) < 2e-2
    assert np.max(np.abs(to_np64(lse2) - ref_lse)) < 2e-2


# ------------------------------------------------------------------ masks
def test_visibility_export_bit_exact():
    banner("visibility predicate export vs oracle (empty slots, multi-block queries)")
    rng = np.random.default_rng(3)
    g, o = make_pair(300, 1, 64, "bf16", 0.0, first_slot=290)
    for b, n in enumerate([40, 70, 33]):
        write_both(g, o, rng, n, 10 * b, b * 2)  # blocks 0, 2, 4
        g.advance(n)
        o.advance(n)
    for n_q, b0, bl in [(1, 0, 1), (90, 0, 20), (300, 1, 7), (64, 4, 64), (17, -3, 5)]:
        m = g.visibility(n_q, b0, bl).cpu().numpy()
        vis, earlier = visibility(o.slot_block, query_blocks(n_q, b0, bl))
        want = np.where(earlier, 2, np.where(vis, 1, 0))
        assert np.array_equal(m, want), (n_q, b0, bl)


def _tile_classes_ref(slot_block, n_q, q_block0, q_block_len, cache_bias, same):
    """Half-tile classes from the visibility definition: for each 32-query wave,
    128-slot tile and half-tile (slots 32 g + 16 h + 0..15 of the tile), bit 1
    if some pair is visible, 2 if the half-tile has an occupied slot and every
    pair with an occupied slot is visible with one bias value (or the bias is
    0), 4 if that value is the bias on every such pair.  Empty slots need no
    mask: the kernel gives them probability 0 through its factor table."""
    N = len(slot_block)
    n_t, n_w = -(-N // 128), -(-n_q // 32)
    sb = np.full(n_t * 128, -1, dtype=np.int64)
    sb[:N] = slot_block
    vis, earlier = visibility(sb, query_blocks(n_q, q_block0, q_block_len), "same" if same else "causal")
    bias_zero = same or cache_bias == 0.0
    out = np.zeros((n_w, n_t, 2), dtype=np.uint8)
    for w in range(n_w):
        qs = slice(32 * w, min(32 * w + 32, n_q))
        for t in range(n_t):
            for h in range(2):
                cols = [128 * t + 32 * g + 16 * h + i for g in range(4) for i in range(16)]
                occ = [c for c in cols if sb[c] != -1]
                v, e = vis[qs][:, occ], earlier[qs][:, occ]
                fast = bool(occ) and bool(v.all()) and (bool(e.all()) or not e.any() or bias_zero)
                out[w, t, h] = int(v.any()) | (int(fast) << 1) | (int(fast and e.all()) << 2)
    return out


def test_tile_class_export_matches_visibility():
    """The FP8 attention kernel's half-tile classes (the decision that skips the
    per-score mask), exported through rc_debug_tile_classes and computed with
    the kernel's own summary and rules, against the visibility definition:
    exact under the block-causal mask; under the same-block mask "may be
    visible" is a superset and "fast" exact."""
    banner("FP8 tile classes vs visibility (wrap, partial tiles, empty slots, multi-block waves)")
    rng = np.random.default_rng(11)
    cases = 0
    # ring A: 300 slots, written from slot 290 (wraps), blocks 0, 2, 4, empty slots left
    g, o = make_pair(300, 1, 64, "bf16", 0.0, first_slot=290)
    for b, n in enumerate([40, 70, 33]):
        write_both(g, o, rng, n, 10 * b, b * 2)
        g.advance(n)
        o.advance(n)
    # ring B: 1,000 FP8 slots, chunks of 96 in blocks 0..11 (wraps, the oldest evicted)
    gb, ob = make_pair(1000, 2, 128, "fp8", 10000.0, first_slot=700)
    for b in range(12):
        write_both(gb, ob, rng, 96, 96 * b, b)
        gb.advance(96)
        ob.advance(96)
    for ring_g, ring_o in ((g, o), (gb, ob)):
        for n_q, b0, bl in [(1, 0, 1), (90, 0, 20), (300, 1, 7), (64, 4, 64), (17, -3, 5), (96, 11, 96),
                            (200, 9, 40)]:
            for bias in (0.0, -0.5):
                for same in (False, True):
                    got = ring_g.tile_classes(n_q, b0, bl, bias, same).cpu().numpy()
                    want = _tile_classes_ref(ring_o.slot_block, n_q, b0, bl, bias, same)
                    assert got.shape == want.shape
                    if same:
                        assert np.array_equal(got & 6, want & 6), (n_q, b0, bl, bias)
                        assert np.all((got & 1) >= (want & 1)), (n_q, b0, bl, bias)
                    else:
                        assert np.array_equal(got, want), (n_q, b0, bl, bias)
                    cases += 1
    print(f"  {cases} cases", flush=True)


# ------------------------------------------------------------------ long run
def test_longrun_scaled_schedule():
    """The long-run schedule scaled down: 14 chunks over a 3-chunk ring, a
    position reset every 5 chunks (delta rebases the oldest cached position
    to 0), a bias ramp 0, -2, -4, -2, 0 over chunks 2..6, 2 denoising passes
    per chunk.  Bookkeeping is compared every chunk, attention on every
    chunk's last pass."""
    banner("long run (scaled): 14 chunks, resets every 5, bias ramp, 2 passes")
    from oracle.schedule import bias_at
    rng = np.random.default_rng(WORKLOADS["longrun"].seed)
    N, H, d, n = 300, 4, 128, 100
    g, o = make_pair(N, H, d, "fp8", 10000.0)
    pos = 0
    worst = 0.0
    for t in range(14):
        if t > 0 and t % 5 == 0:
            oldest = int(o.slot_pos[o.slot_block != -1].min())
            g.rerotate(-oldest)
            o.rerotate(-oldest)
            pos -= oldest
        beta = bias_at(t, n_ramps=1, first=2, spacing=1)
        for _ in range(2):
            write_both(g, o, rng, n, pos, t)
            qt, q = inputs(rng, "fp8", (n, H, d))
            out = g.attention(qt, pos, t, n, beta)
        c = gpu_cache(g)
        assert c["state"] == o.state()
        assert np.array_equal(c["slot_block"], o.slot_block)
        assert np.array_equal(c["slot_pos"][o.slot_block != -1], o.slot_pos[o.slot_block != -1])
        ref, _ = ring_attention(oracle_from_gpu(g, 10000.0), q, pos, t, n, beta)
        err, _ = assert_attention_close(out, ref, "fp8")
        ref_own, _ = ring_attention(o, q, pos, t, n, beta)
        assert_attention_close(out, ref_own, "fp8")
        worst = max(worst, err)
        g.advance(n)
        o.advance(n)
        pos += n
    print(f"  worst max-abs {worst:.3e}", flush=True)
