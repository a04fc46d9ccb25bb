"""GPU parity of the scored content memory: rc_key_mass and
rc_cache_write_scored through the C ABI against the float64 oracle.

* Key mass: the GPU's mass (FP8 products, the attention's lse) against the
  oracle's exact column sums of the softmax over the GPU's own cache, with
  the tolerance below; rows of the softmax sum to one, so the total mass of
  a head is the number of queries; the result is reproducible to the bit.
* Scored writes: synthetic scores (seeded; uniform, heavily tied, and with
  zero rows) given to both sides; the choice is an integer decision taken in
  float64 on both sides by the same rule, so the memory's contents and all
  bookkeeping must match exactly (codes as for any cache write).

Key mass tolerance.  Every probability carries the FP8 rounding of its
query (one scale per 32 queries) and key (3 mantissa bits each: relative
error up to 2^-4 per element, averaging over d terms of the dot product) and
the attention's own lse (which has the same kind of error); at unit-variance
inputs the logits move by ~1e-2, so each p moves by ~1 % and the mass of a
slot, a sum of many such terms with independent errors, by less (measured:
relative L2 4e-3, worst entry 8e-3).  Gate: relative L2 error over all
(head, slot) entries <= 1.5e-2 and every entry within 2.5e-2 * (1 + its
value).  Real bugs (a dropped bias, a wrong block, a wrong row's lse) move
entries by tens of percent.
"""
import sys

import numpy as np
import pytest
import torch

from autoregressive_video_diffusion_ring_amd import Ring
from oracle.attention import ring_attention
from oracle.memory import ring_key_mass
from oracle.ring import Ring as OracleRing

from gpu_helpers import (DEV, assert_attention_close, compare_cache, gpu_cache, inputs, oracle_from_gpu, oracle_rows,
                         rel_l2, to_np64)

pytestmark = pytest.mark.gpu


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU", allow_module_level=True)


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def make_pair(N, H, d, kv, n_anchor=0, n_memory=0):
    return (Ring(N, H, d, kv, 10000.0, n_anchor=n_anchor, n_memory=n_memory, device=DEV),
            OracleRing(N, H, d, kv, 10000.0, n_anchor=n_anchor, n_memory=n_memory))


def write_both(g, o, rng, n, pos0, blk, scores=None, gamma=1.0):
    kt, k = inputs(rng, g.kv_name, (n, g.H, g.d))
    vt, v = inputs(rng, g.kv_name, (n, g.H, g.d))
    if scores is None:
        g.write(kt, vt, pos0, blk)
        o.write(k, v, n, pos0, blk)
    else:
        g.write_scored(kt, vt, pos0, blk, torch.from_numpy(scores).to(DEV), gamma)
        o.write_scored(k, v, n, pos0, blk, scores[:, :g.N], gamma)


MASS_REL_L2, MASS_ENTRY = 1.5e-2, 2.5e-2


def check_mass(got, ref):
    got = got[:, :ref.shape[1]]
    r = rel_l2(got, ref)
    worst = float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))
    print(f"  mass rel-L2 {r:.3e}, worst entry {worst:.3e}", flush=True)
    assert r <= MASS_REL_L2 and worst <= MASS_ENTRY


# ------------------------------------------------------------------ key mass
@pytest.mark.parametrize("d", [128, 64])
def test_key_mass_single_block(d):
    banner(f"key mass: fp8 d={d} N=700 H=4, 500 history + 150 current, bias -0.5")
    rng = np.random.default_rng(51)
    N, H = 700, 4
    g, o = make_pair(N, H, d, "fp8")
    write_both(g, o, rng, 500, 0, 0)
    g.advance(500)
    o.advance(500)
    write_both(g, o, rng, 150, 500, 1)
    qt, q = inputs(rng, "fp8", (150, H, d))
    lse = torch.empty((H, 150), dtype=torch.float32, device=DEV)
    g.attention(qt, 500, 1, 150, -0.5, lse=lse)
    mass = g.key_mass(qt, 500, 1, 150, -0.5, lse)
    got = to_np64(mass)
    ref = ring_key_mass(oracle_from_gpu(g, 10000.0), q, 500, 1, 150, -0.5)
    check_mass(got, ref)
    assert np.allclose(got.sum(axis=1), 150.0, rtol=2e-2)
    assert np.all(got[:, N:] == 0)
    again = g.key_mass(qt, 500, 1, 150, -0.5, lse)           # a fresh buffer: same bits
    assert torch.equal(mass, again)
    g.key_mass(qt, 500, 1, 150, -0.5, lse, mass=again)       # accumulates
    assert torch.equal(again, 2 * mass)


def test_key_mass_multiblock_ragged():
    """Queries of three blocks of 50 (32-query tiles straddle block edges),
    a wrapped ring with empty slots, bias -0.5."""
    banner("key mass: fp8 d=128 N=300 H=3, 150 queries in blocks of 50, wrapped ring")
    rng = np.random.default_rng(52)
    N, H, d = 300, 3, 128
    g = Ring(N, H, d, "fp8", 10000.0, first_slot=250, device=DEV)
    o = OracleRing(N, H, d, "fp8", 10000.0, first_slot=250)
    for b, (n, p0) in enumerate([(60, 1000), (70, 1060), (50, 1130)]):
        write_both(g, o, rng, n, p0, b)
        g.advance(n)
        o.advance(n)
    qt, q = inputs(rng, "fp8", (150, H, d))
    lse = torch.empty((H, 150), dtype=torch.float32, device=DEV)
    g.attention(qt, 1060, 1, 50, -0.5, lse=lse)
    got = to_np64(g.key_mass(qt, 1060, 1, 50, -0.5, lse))
    ref = ring_key_mass(oracle_from_gpu(g, 10000.0), q, 1060, 1, 50, -0.5)
    check_mass(got, ref)
    # queries of block 3 see no key of their own block; every query sees some key
    assert np.allclose(got.sum(axis=1), 150.0, rtol=2e-2)


def test_key_mass_slot_ranges():
    """rc_key_mass_slots: the mass of the listed slots equals rc_key_mass's,
    bit for bit, and every other entry keeps its old value.  Ranges as the
    scored write uses them (memory slots and a write range that wraps), on a
    wrapped ring with empty slots."""
    banner("key mass over slot ranges: fp8 d=128 N=1500 H=3, ranges that wrap and straddle groups")
    rng = np.random.default_rng(54)
    N, H, d = 1500, 3, 128
    g = Ring(N, H, d, "fp8", 10000.0, first_slot=1300, device=DEV)
    for b, (n, p0) in enumerate([(400, 0), (500, 400), (300, 900)]):
        kt, _ = inputs(rng, "fp8", (n, H, d))
        vt, _ = inputs(rng, "fp8", (n, H, d))
        g.write(kt, vt, p0, b)
        g.advance(n)
    qt, _ = inputs(rng, "fp8", (300, H, d))
    lse = torch.empty((H, 300), dtype=torch.float32, device=DEV)
    g.attention(qt, 900, 2, 300, -0.5, lse=lse)
    full = g.key_mass(qt, 900, 2, 300, -0.5, lse)
    for ranges in ([(1300, 1500), (0, 37)], [(5, 6)], [(0, 1500)], [(511, 513), (1000, 1024), (1100, 1200)]):
        sentinel = torch.full_like(full, 7.0)
        got = g.key_mass(qt, 900, 2, 300, -0.5, lse, mass=sentinel.clone(), ranges=ranges)
        inside = torch.zeros(full.shape[1], dtype=torch.bool, device=DEV)
        for lo, hi in ranges:
            inside[lo:hi] = True
        assert torch.equal(got[:, inside], full[:, inside] + 7.0), ranges
        assert torch.all(got[:, ~inside] == 7.0), ranges


def test_key_mass_stream_full_size():
    """The streaming shape (757 queries over 5,788 FP8 slots, 40 heads); the
    oracle checks four of the heads."""
    banner("key mass: streaming shape 757 x 5788 fp8, 40 heads (oracle on heads 0-3)")
    rng = np.random.default_rng(53)
    N, H, d = 5788, 40, 128
    g, o = make_pair(N, H, d, "fp8")
    write_both(g, o, rng, 5031, 0, 0)
    g.advance(5031)
    o.advance(5031)
    write_both(g, o, rng, 757, 5031, 1)
    qt, q = inputs(rng, "fp8", (757, H, d))
    lse = torch.empty((H, 757), dtype=torch.float32, device=DEV)
    g.attention(qt, 5031, 1, 757, 0.0, lse=lse)
    got = to_np64(g.key_mass(qt, 5031, 1, 757, 0.0, lse))
    assert np.allclose(got.sum(axis=1), 757.0, rtol=2e-2)
    full = oracle_from_gpu(g, 10000.0)
    sub = OracleRing.from_arrays(kv_dtype="fp8", rope_base=10000.0, k=full.k[:4], v=full.v[:4],
                                 k_scale=full.k_scale[:4], v_scale=full.v_scale[:4], slot_pos=full.slot_pos,
                                 slot_block=full.slot_block, state=full.state())
    ref = ring_key_mass(sub, q[:, :4], 5031, 1, 757, 0.0)
    check_mass(got[:4], ref)


# ------------------------------------------------------------------ scored writes
def scores(rng, kind, H, v_ld):
    if kind == "ties":
        s = rng.integers(0, 3, size=(H, v_ld)).astype(np.float32)
    else:
        s = rng.uniform(0, 1, size=(H, v_ld)).astype(np.float32)
    if kind == "zeros":
        s[:, rng.random(v_ld) < 0.3] = 0.0
    return s


@pytest.mark.parametrize("kv,d,N,A,M,n,H,chunks,gamma,kind", [
    ("fp8", 128, 300, 20, 60, 40, 3, 12, 1.0, "uniform"),
    ("fp8", 128, 300, 20, 60, 40, 3, 12, 0.5, "ties"),
    ("fp8", 64, 257, 0, 45, 33, 2, 14, 0.25, "zeros"),
    ("bf16", 64, 200, 16, 50, 30, 3, 12, 0.75, "ties"),
    ("fp8", 128, 5788, 757, 1024, 757, 8, 8, 0.9, "uniform"),   # the streaming shape
])
def test_scored_write_parity(kv, d, N, A, M, n, H, chunks, gamma, kind):
    banner(f"scored write: {kv} d={d} N={N} A={A} M={M} chunks of {n}, H={H}, gamma {gamma}, {kind} scores")
    rng = np.random.default_rng(61)
    g, o = make_pair(N, H, d, kv, n_anchor=A, n_memory=M)
    v_ld = g.v_ld
    for b in range(chunks):
        sc = scores(rng, kind, H, v_ld)
        write_both(g, o, rng, n, n * b, b, sc, gamma)
        compare_cache(gpu_cache(g), o, kv)
        # a second pass of the chunk: the memory does not change
        write_both(g, o, rng, n, n * b, b, scores(rng, kind, H, v_ld), gamma)
        compare_cache(gpu_cache(g), o, kv)
        g.advance(n)
        o.advance(n)
    assert o.n_mem == M, "the case must fill the memory"
    # attention over anchor, sliding part and memory
    qt, q = inputs(rng, kv, (n, H, d))
    out = g.attention(qt, n * chunks, chunks, n, -0.5)
    rows = np.r_[0:n:max(1, n // 40), n - 1]
    ref, _ = oracle_rows(oracle_from_gpu(g, 10000.0), q, rows, n * chunks, chunks, n, -0.5)
    assert_attention_close(out, ref, kv, rows=rows)


def test_scored_stream_with_gpu_mass():
    """Scores from the GPU's own key mass, fed back into the next chunk's
    scored write (the intended use): bookkeeping follows the oracle's
    closed forms and every cached token appears once."""
    banner("scored stream: fp8 d=128 N=1000 A=100 M=300, chunks of 100, mass-driven")
    rng = np.random.default_rng(62)
    N, A, M, n, H, d = 1000, 100, 300, 100, 4, 128
    g = Ring(N, H, d, "fp8", 10000.0, n_anchor=A, n_memory=M, device=DEV)
    mass = torch.zeros((H, g.v_ld), dtype=torch.float32, device=DEV)
    E = N - M
    evicted = 0
    for b in range(14):
        kt, _ = inputs(rng, "fp8", (n, H, d))
        vt, _ = inputs(rng, "fp8", (n, H, d))
        before = g.state()[1]
        g.write_scored(kt, vt, n * b, b, mass, 0.5)
        evicted += before - g.state()[1]
        qt, _ = inputs(rng, "fp8", (n, H, d))
        lse = torch.empty((H, n), dtype=torch.float32, device=DEV)
        g.attention(qt, n * b, b, n, -0.5, lse=lse)
        mass.zero_()
        g.key_mass(qt, n * b, b, n, -0.5, lse, mass=mass)
        g.advance(n)
        c = gpu_cache(g)
        assert c["state"][5] == min(M, evicted)
        w = c["slot_block"] != -1
        toks = list(zip(c["slot_pos"][w].tolist(), c["slot_block"][w].tolist()))
        assert len(toks) == len(set(toks))
        assert np.array_equal(c["slot_pos"][:A], np.arange(A))
        total = n * (b + 1)
        fifo = np.sort(c["slot_pos"][A:E][c["slot_block"][A:E] != -1])
        assert np.array_equal(fifo, np.arange(max(A, total - (E - A)), total))
        mem = c["slot_pos"][E:][c["slot_block"][E:] != -1]
        assert np.all((mem >= A) & (mem < max(A, total - (E - A))))
