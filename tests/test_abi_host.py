"""Host-side checks of the C ABI that need no GPU.

* librc.so loads and exports every function include/rc.h declares.
* rc_ring_advance and the host bookkeeping of rc_cache_write's checks are
  bit-exact against the oracle's ring (rc_ring_advance is host only; the
  argument and state checks run before anything is enqueued, so they are
  exercised here with placeholder device pointers that are never touched).
* Every rejected call leaves the host state unchanged.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from autoregressive_video_diffusion_ring_amd import _lib
from autoregressive_video_diffusion_ring_amd._lib import (RC_BF16, RC_ERR_ARG, RC_ERR_STATE, RC_ERR_UNSUPPORTED,
                                                          RC_FP8_E4M3, RC_F32, RC_OK, RcRing, lib)
from oracle.ring import Ring as OracleRing, RingStateError

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "rc.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rc_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_header_symbol():
    names = header_functions()
    assert "rc_chunk_attention" in names and "rc_cache_write" in names and len(names) >= 10
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with rc.h"


def test_struct_layout_matches_c():
    # int32 x 4, float, int32 x 2, then six pointers at 8-byte alignment, then 5 int32
    assert RcRing.n_anchor.offset == 24
    assert RcRing.k.offset == 32 and RcRing.slot_block.offset == 72
    assert RcRing.head.offset == 80 and RcRing.cur_block.offset == 96
    assert ctypes.sizeof(RcRing) == 104


FAKE = 1 << 20  # aligned placeholder address; never dereferenced by the checks below


def fake_ring(N, H=2, d=64, kv=RC_FP8_E4M3, head=0, n_hist=0, n_cur=0, n_anchor=0):
    r = RcRing()
    r.n_slots, r.n_heads, r.head_dim, r.kv_dtype = N, H, d, kv
    r.n_anchor = n_anchor
    r.rope_base = 10000.0
    r.v_ld = lib().rc_ring_v_ld(N)
    r.k = r.v = r.k_scale = r.v_scale = r.slot_pos = r.slot_block = FAKE
    r.head, r.n_hist, r.n_cur = head, n_hist, n_cur
    return r


def state(r):
    return (r.head, r.n_hist, r.n_cur, r.cur_pos0, r.cur_block)


def test_v_ld_and_sizes():
    L = lib()
    assert [L.rc_ring_v_ld(n) for n in (1, 63, 64, 65, 5788, 11520)] == [64, 64, 64, 128, 5824, 11520]
    out = (ctypes.c_size_t * 6)()
    assert L.rc_ring_sizes(5788, 40, 128, RC_FP8_E4M3, out) == RC_OK
    assert list(out) == [40 * 5824 * 128, 40 * 128 * 5824, 40 * 5824 * 4, 40 * 5824 * 4, 5824 * 4, 5824 * 4]
    assert L.rc_ring_sizes(96, 2, 64, RC_F32, out) == RC_OK
    assert list(out) == [2 * 128 * 64 * 4, 2 * 64 * 128 * 4, 0, 0, 128 * 4, 128 * 4]
    assert L.rc_ring_sizes(96, 2, 96, RC_BF16, out) == RC_ERR_UNSUPPORTED
    assert L.rc_ring_sizes(0, 2, 64, RC_BF16, out) == RC_ERR_ARG
    assert L.rc_ring_sizes(10, 2, 64, 7, out) == RC_ERR_ARG


@pytest.mark.parametrize("N,n,h0,chunks,A", [(5788, 757, 5031, 30, 0), (96, 32, 0, 9, 0), (10, 10, 3, 4, 0),
                                             (7, 3, 6, 12, 0), (5788, 757, 0, 30, 757), (10, 3, 0, 12, 3),
                                             (10, 3, 0, 12, 4), (7, 1, 0, 20, 6)])
def test_advance_matches_oracle(N, n, h0, chunks, A):
    """Host bookkeeping of write + advance, bit-exact against the oracle,
    with and without pinned anchor slots.

    The write's device work cannot run here, so the write's host update is
    replayed by hand exactly as rc_cache_write applies it after a successful
    launch; rc_ring_advance itself runs in the library."""
    L = lib()
    r = fake_ring(N, head=h0, n_anchor=A)
    o = OracleRing(N, 1, 2, "f32", 0.0, first_slot=h0, n_anchor=A)
    z = np.zeros((n, 1, 2))
    for t in range(chunks):
        o.write(z, z, n, n * t, t)
        r.n_hist = min(r.n_hist, N - n)
        r.n_cur, r.cur_pos0, r.cur_block = n, n * t, t
        assert state(r) == o.state()
        assert L.rc_ring_advance(ctypes.byref(r), n) == RC_OK
        o.advance(n)
        assert state(r) == o.state()


def test_advance_rejections_leave_state():
    L = lib()
    r = fake_ring(100, head=5, n_hist=20, n_cur=0)
    before = state(r)
    assert L.rc_ring_advance(ctypes.byref(r), 10) == RC_ERR_STATE
    assert "n_cur" in L.rc_last_error().decode()
    r.n_cur = 10
    assert L.rc_ring_advance(ctypes.byref(r), 9) == RC_ERR_STATE
    assert state(r) == before[:2] + (10,) + before[3:]
    r.head = 100  # corrupt
    assert L.rc_ring_advance(ctypes.byref(r), 10) == RC_ERR_STATE
    assert L.rc_ring_advance(None, 10) == RC_ERR_ARG


def test_write_argument_and_state_checks():
    L = lib()
    r = fake_ring(100, head=5, n_hist=20)
    r.n_cur, r.cur_pos0, r.cur_block = 10, 50, 3
    before = state(r)
    bad = [
        (FAKE, FAKE, 0, 50, 3, RC_ERR_ARG),      # n_new < 1
        (FAKE, FAKE, 101, 50, 3, RC_ERR_ARG),    # n_new > N
        (0, FAKE, 10, 50, 3, RC_ERR_ARG),        # NULL k_new
        (FAKE + 4, FAKE, 10, 50, 3, RC_ERR_ARG), # misaligned
        (FAKE, FAKE, 10, 50, -1, RC_ERR_ARG),    # negative block
        (FAKE, FAKE, 9, 50, 3, RC_ERR_STATE),    # rewrite with another n
        (FAKE, FAKE, 10, 51, 3, RC_ERR_STATE),   # rewrite at another position
        (FAKE, FAKE, 10, 50, 4, RC_ERR_STATE),   # rewrite with another block
    ]
    for k, v, n, pos0, blk, want in bad:
        got = L.rc_cache_write(ctypes.byref(r), k, v, n, pos0, blk, None)
        assert got == want, (n, pos0, blk, got, L.rc_last_error())
        assert state(r) == before
    ra = fake_ring(100, n_anchor=30)
    assert L.rc_cache_write(ctypes.byref(ra), FAKE, FAKE, 71, 0, 0, None) == RC_ERR_ARG  # > N - n_anchor
    assert "n_anchor" in L.rc_last_error().decode()
    ra.n_anchor = 100
    assert L.rc_cache_write(ctypes.byref(ra), FAKE, FAKE, 1, 0, 0, None) == RC_ERR_ARG
    ra.n_anchor = -1
    assert L.rc_cache_write(ctypes.byref(ra), FAKE, FAKE, 1, 0, 0, None) == RC_ERR_ARG
    assert state(ra) == (0, 0, 0, 0, 0)
    r2 = fake_ring(100)
    r2.v_ld = 100  # wrong leading dimension
    assert L.rc_cache_write(ctypes.byref(r2), FAKE, FAKE, 1, 0, 0, None) == RC_ERR_ARG
    r3 = fake_ring(100, kv=RC_FP8_E4M3)
    r3.k_scale = 0
    assert L.rc_cache_write(ctypes.byref(r3), FAKE, FAKE, 1, 0, 0, None) == RC_ERR_ARG


def test_attention_argument_checks():
    L = lib()
    r = fake_ring(100)
    args = dict(q=FAKE, n_q=10, pos=0, b0=0, bl=10, bias=0.0, scale=0.0, out=FAKE, ws=0, wsb=0)

    def call(**kw):
        a = dict(args, **kw)
        return L.rc_chunk_attention(ctypes.byref(r), a["q"], a["n_q"], a["pos"], a["b0"], a["bl"], a["bias"],
                                    a["scale"], a["out"], None, a["ws"], a["wsb"], None)
    assert call(n_q=0) == RC_ERR_ARG
    assert call(bl=0) == RC_ERR_ARG
    assert call(q=0) == RC_ERR_ARG
    assert call(out=FAKE + 2) == RC_ERR_ARG
    assert call(scale=-1.0) == RC_ERR_ARG
    assert call(scale=float("nan")) == RC_ERR_ARG
    assert call(bias=float("nan")) == RC_ERR_ARG
    assert call(wsb=64) == RC_ERR_ARG
    r.head_dim = 96
    assert call() == RC_ERR_UNSUPPORTED
    f = fake_ring(100, d=128, kv=RC_F32)
    assert L.rc_chunk_attention(ctypes.byref(f), FAKE, 10, 0, 0, 10, 0.0, 0.0, FAKE, None, 0, 0,
                                None) == RC_ERR_UNSUPPORTED


def test_rerotate_needs_rope():
    L = lib()
    r = fake_ring(100)
    r.rope_base = 0.0
    assert L.rc_cache_rerotate(ctypes.byref(r), 5, None) == RC_ERR_ARG
    r.rope_base = -1.0
    assert L.rc_cache_rerotate(ctypes.byref(r), 5, None) == RC_ERR_ARG


def test_init_checks():
    L = lib()
    r = fake_ring(100)
    assert L.rc_ring_init(ctypes.byref(r), 100, None) == RC_ERR_ARG
    assert L.rc_ring_init(ctypes.byref(r), -1, None) == RC_ERR_ARG
    r.slot_block = 0
    assert L.rc_ring_init(ctypes.byref(r), 0, None) == RC_ERR_ARG
    a = fake_ring(100, n_anchor=20)
    assert L.rc_ring_init(ctypes.byref(a), 5, None) == RC_ERR_ARG   # an anchored ring starts at 0
    a.n_anchor = 100
    assert L.rc_ring_init(ctypes.byref(a), 0, None) == RC_ERR_ARG


def test_advance_checks_anchor():
    L = lib()
    r = fake_ring(10, n_anchor=10, n_cur=3)
    assert L.rc_ring_advance(ctypes.byref(r), 3) == RC_ERR_ARG
    r.n_anchor = 3
    r.head = 9
    assert L.rc_ring_advance(ctypes.byref(r), 3) == RC_OK
    assert state(r)[:3] == (5, 3, 0)    # 9 -> 3 + (9 + 3 - 10)
