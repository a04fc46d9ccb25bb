"""GPU parity of the fused QKV projection + cache write (rc_qkv_project_write)
against the float64 oracle (oracle/projection.py, then the oracle ring's
write).

Inputs: x bf16 N(0,1); W as uniformly random finite e4m3 codes with float32
row scales (synthetic weights), both fed to the two sides as the same bytes.

Tolerances.  The matrix core forms the FP8 products exactly but sums each
group of 64 of them in reduced precision: a one-wave probe with random
e4m3 codes measured errors up to 2^-12.7 of the group's sum of |terms| (and
2^-14 for operands of a narrower range); the groups are then added in
float32.  The oracle sums in float64.  So q, rounded to bfloat16, must lie
within one bf16 unit of the correctly rounded reference plus 2^-11 of the
sum of |terms| (which matters only where terms cancel); cached codes within one FP8 step (a quotient near
a rounding boundary can fall either way, and a value that cancels to almost
nothing can move several of its small steps): dequantized, within one step
plus the same bound, and scales within 2^-10.  Bookkeeping (slots, positions, blocks, state) is
exact.
"""
import sys

import numpy as np
import pytest
import torch

from autoregressive_video_diffusion_ring_amd import Ring
from oracle import e4m3
from oracle.projection import qkv_project, quantize_tokens
from oracle.ring import Ring as OracleRing, round_bf16
from synthetic_inputs import e4m3_codes, normal_bf16

from gpu_helpers import DEV, gpu_cache, to_np64

pytestmark = pytest.mark.gpu


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU", allow_module_level=True)


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def weights(rng, H, d, C):
    codes = e4m3_codes(rng, (3 * H * d, C))
    scale = rng.uniform(0.5, 1.0, size=3 * H * d).astype(np.float32) / np.float32(64.0 * np.sqrt(C))
    return codes, scale


def check_cache(c, o, written, bound_k, bound_v):
    """Bookkeeping exact; cached K and V within one FP8 step of the oracle's
    value plus the propagated summation bound (per token, head, column)."""
    assert c["state"] == o.state()
    assert np.array_equal(c["slot_block"], o.slot_block)
    w = o.slot_block != -1
    assert np.array_equal(c["slot_pos"][w], o.slot_pos[w])
    for name, sname, bound in (("k", "k_scale", bound_k), ("v", "v_scale", bound_v)):
        go, oo = c[name][:, written], getattr(o, name)[:, written]
        gs, os_ = c[sname][:, written], getattr(o, sname)[:, written]
        gval = e4m3.dequantize(go, gs)
        oval = e4m3.dequantize(oo, os_)
        mag = (oo & 0x7F).astype(np.int64)
        up = e4m3.decode(np.minimum(mag + 1, 0x7E).astype(np.uint8)) - e4m3.decode(mag.astype(np.uint8))
        down = e4m3.decode(mag.astype(np.uint8)) - e4m3.decode(np.maximum(mag - 1, 0).astype(np.uint8))
        step = np.maximum(up, down) * os_[..., None]   # the wider gap next to the code (0x7E has none above)
        dev = np.abs(gval - oval)
        tol = step + bound
        dist = e4m3.ulp_distance(go, oo)
        wi = np.unravel_index(np.argmax(dev / tol), dev.shape)
        bad = dev > tol
        print(f"  {name}: codes differing {np.count_nonzero(dist) / dist.size:.2e} (max {dist.max()} steps); "
              f"worst value deviation {np.max(dev / tol):.2f} of allowed at (h, slot index, col) {wi}: "
              f"gpu {gval[wi]:.4e} ref {oval[wi]:.4e} step {step[wi]:.2e} bound {bound[wi]:.2e}; "
              f"over: {np.count_nonzero(bad)} at heads {sorted(set(np.nonzero(bad)[0].tolist()))[:8]} "
              f"slot idx {sorted(set(np.nonzero(bad)[1].tolist()))[:8]} cols {sorted(set(np.nonzero(bad)[2].tolist()))[:8]}",
              flush=True)
        assert np.all(dev <= tol)
        assert np.all(np.abs(gs.astype(np.float64) - os_) <= 2.0 ** -10 * os_ + 1e-30)


def summation_bounds(x, wc, ws, H, d, order, written):
    """2^-11 of the sum of |terms| of every k and v output (k: both members of
    its rotation pair, which the rotation mixes), laid out as the cache
    [H][slot][d] restricted to the written slots."""
    HD = H * d
    xd = e4m3.dequantize(*quantize_tokens(x))
    out = []
    for part in (1, 2):
        wd = e4m3.dequantize(wc[part * HD:(part + 1) * HD], ws[part * HD:(part + 1) * HD])
        a = (np.abs(xd) @ np.abs(wd).T).reshape(x.shape[0], H, d)
        if part == 1:
            a = np.repeat(a.reshape(x.shape[0], H, d // 2, 2).sum(-1), 2, axis=-1)
        cache = np.zeros((H, len(written), d))
        pos = {s: i for i, s in enumerate(written)}
        for t, s in enumerate(order):
            cache[:, pos[int(s)], :] = a[t]
        out.append(2.0 ** -11 * cache)
    return out


@pytest.mark.parametrize("n,C,H,N,head0,hist,anchor,memory", [
    (100, 256, 2, 300, 250, 0, 0, 0),         # ragged token tile, a write that wraps
    (1, 128, 1, 64, 10, 0, 0, 0),             # one token, the narrowest input (two k steps)
    (385, 1024, 3, 1200, 1000, 200, 0, 0),    # a second token tile holding one token; wrap after history
    (40, 8320, 2, 200, 0, 0, 0, 0),           # input rows wider than one wave holds (two-pass quantiser)
    (200, 256, 2, 600, 0, 400, 50, 100),      # anchored ring with a content memory: the write wraps
                                              # from the memory's first slot (500) to slot 50
    (757, 5120, 40, 5788, 0, 5031, 0, 0),     # the streaming shape: 757 new tokens after 5,031 of history
])
def test_qkv_project_write(n, C, H, N, head0, hist, anchor, memory):
    banner(f"qkv projection + write: n={n} C={C} H={H} N={N} head0={head0} history {hist} "
           f"anchor {anchor} memory {memory}")
    rng = np.random.default_rng(71)
    d = 128
    g = Ring(N, H, d, "fp8", 10000.0, first_slot=head0, n_anchor=anchor, n_memory=memory, device=DEV)
    o = OracleRing(N, H, d, "fp8", 10000.0, first_slot=head0, n_anchor=anchor, n_memory=memory)
    if hist:
        kb, k = normal_bf16(rng, (hist, H, d))
        vb, v = normal_bf16(rng, (hist, H, d))
        g.write(torch.from_numpy(kb.view(np.int16)).to(DEV).view(torch.bfloat16),
                torch.from_numpy(vb.view(np.int16)).to(DEV).view(torch.bfloat16), 0, 0)
        o.write(k, v, hist, 0, 0)
        g.advance(hist)
        o.advance(hist)
    xb, x = normal_bf16(rng, (n, C))
    wc, ws = weights(rng, H, d, C)
    xt = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    q = g.project_write(xt, torch.from_numpy(wc).to(DEV), torch.from_numpy(ws).to(DEV), hist, 1)
    q_ref, k_ref, v_ref = qkv_project(x, wc, ws, H, d)
    o.write(k_ref, v_ref, n, hist, 1)
    qg = to_np64(q)
    ref_b = round_bf16(q_ref)   # correctly rounded reference; the GPU may land on its neighbour
    ulp = np.where(ref_b != 0, 2.0 ** (np.floor(np.log2(np.abs(np.where(ref_b != 0, ref_b, 1.0)))) - 7), 2.0 ** -133)
    # the FP8 matrix core sums each group of 64 products in reduced precision:
    # up to 2^-12.7 of the group's sum of |terms| (measured with random codes);
    # the bound allows 2^-11 of the sum of |terms| (large only where terms cancel)
    xd = e4m3.dequantize(*quantize_tokens(x))
    wd = e4m3.dequantize(wc[:H * d], ws[:H * d])
    absum = (np.abs(xd) @ np.abs(wd).T).reshape(n, H, d)
    tol = ulp + 2.0 ** -11 * absum
    dev = np.abs(qg - ref_b)
    i = np.unravel_index(np.argmax(dev / tol), dev.shape)
    print(f"  q: worst {dev[i]:.3e} of allowed {tol[i]:.3e} (ref {q_ref[i]:.3e}, sum|terms| {absum[i]:.3e}); "
          f"differing from the rounded reference: {np.count_nonzero(dev) / dev.size:.2e}", flush=True)
    assert np.all(dev <= tol)
    written = np.nonzero(o.slot_block == 1)[0]
    order = o.write_slots(n)            # slot of token i (as [H][slot][d] for the cache)
    bk, bv = summation_bounds(x, wc, ws, H, d, order, written)
    check_cache(gpu_cache(g), o, written, bk, bv)
    # a second pass of the same chunk overwrites the same slots
    xb2, x2 = normal_bf16(rng, (n, C))
    g.project_write(torch.from_numpy(xb2.view(np.int16)).to(DEV).view(torch.bfloat16),
                    torch.from_numpy(wc).to(DEV), torch.from_numpy(ws).to(DEV), hist, 1)
    _, k2, v2 = qkv_project(x2, wc, ws, H, d)
    o.write(k2, v2, n, hist, 1)
    bk, bv = summation_bounds(x2, wc, ws, H, d, order, written)
    check_cache(gpu_cache(g), o, written, bk, bv)
