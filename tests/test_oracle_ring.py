"""Pins for the oracle's ring-cache bookkeeping, write and delta re-rotation.

* Bookkeeping is checked against an independent model (a replay of every
  token ever written into explicit cells, the k-th token going to cell
  (first + k) mod N, or with an anchor of A slots to cell k for k < A and
  A + (k - A) mod (N - A) after) under random call sequences drawn by
  Hypothesis.
* Closed forms: the head after T chunks of n tokens is (h0 + n T) mod N.
* Write: cached values are the rotated inputs up to one quantisation step.
* Delta rotation equals re-encoding at the moved positions: exactly up to
  float32 storage rounding, and within two code steps with FP8 storage.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import e4m3
from oracle.ring import Ring, RingStateError, round_bf16
from oracle.rope import rope


class CellModel:
    """Independent model: a list of all tokens written (the current chunk can
    be rewritten), replayed into N cells."""

    def __init__(self, N, first, A=0):
        self.N, self.first, self.A = N, first, A
        self.committed = []  # (pos, block)
        self.current = []

    def write(self, n, pos0, blk):
        self.current = [(pos0 + i, blk) for i in range(n)]

    def rerotate(self, delta):
        self.committed = [(p + delta, b) for p, b in self.committed]
        self.current = [(p + delta, b) for p, b in self.current]

    def advance(self):
        self.committed += self.current
        self.current = []

    def cell(self, k):
        if k < self.A:
            return k
        return self.A + (self.first + k - self.A) % (self.N - self.A)

    def cells(self):
        pos = {}
        owner = {}
        for k, tok in enumerate(self.committed + self.current):
            c = self.cell(k)
            pos[c] = tok
            owner[c] = k
        return pos, owner

    def expect(self):
        pos, owner = self.cells()
        nc = len(self.committed)
        head = self.cell(nc)
        n_hist = sum(1 for c, k in owner.items() if k < nc)
        slot_pos = np.zeros(self.N, dtype=np.int64)
        slot_block = np.full(self.N, -1, dtype=np.int64)
        for c, (p, b) in pos.items():
            slot_pos[c], slot_block[c] = p, b
        return head, n_hist, len(self.current), slot_pos, slot_block


ops = st.lists(st.tuples(st.sampled_from(["write", "advance", "rerotate", "rewrite"]),
                         st.integers(1, 40), st.integers(-50, 50)), min_size=1, max_size=40)


@settings(max_examples=300, deadline=None)
@given(N=st.integers(1, 40), first=st.integers(0, 39), anchor=st.integers(0, 39), seq=ops)
def test_bookkeeping_matches_cell_model(N, first, anchor, seq):
    # half the cases without an anchor (any first slot), half with one
    A = 0 if anchor % 2 == 0 else (anchor // 2) % N
    first = first % N if A == 0 else 0
    H, d = 1, 2
    ring = Ring(N, H, d, "f32", 0.0, first_slot=first, n_anchor=A)
    model = CellModel(N, first, A)
    pos_next, blk_next = 0, 0
    for op, n, delta in seq:
        n = (n - 1) % (N - A) + 1
        if op == "write" and ring.n_cur == 0:
            z = np.zeros((n, H, d))
            ring.write(z, z, n, pos_next, blk_next)
            model.write(n, pos_next, blk_next)
        elif op == "rewrite" and ring.n_cur > 0:
            m = ring.n_cur
            z = np.ones((m, H, d))
            ring.write(z, z, m, ring.cur_pos0, ring.cur_block)
        elif op == "advance" and ring.n_cur > 0:
            pos_next = ring.cur_pos0 + ring.n_cur
            blk_next += 1
            ring.advance(ring.n_cur)
            model.advance()
        elif op == "rerotate":
            ring.rerotate(delta)
            model.rerotate(delta)
            pos_next += delta
        head, n_hist, n_cur, slot_pos, slot_block = model.expect()
        assert (ring.head, ring.n_hist, ring.n_cur) == (head, n_hist, n_cur)
        assert np.array_equal(ring.slot_block, slot_block)
        written = slot_block != -1
        assert np.array_equal(ring.slot_pos[written], slot_pos[written])


def test_head_closed_form_streaming():
    N, n, h0 = 5788, 757, 5031
    ring = Ring(N, 1, 2, "f32", 0.0, first_slot=h0)
    z = np.zeros((n, 1, 2))
    for T in range(1, 40):
        ring.write(z, z, n, n * (T - 1), T - 1)
        ring.advance(n)
        assert ring.head == (h0 + n * T) % N
        assert ring.n_hist == min(n * T, N)


def test_write_errors_leave_state_unchanged():
    ring = Ring(10, 1, 2, "f32", 0.0)
    z = np.zeros((4, 1, 2))
    ring.write(z, z, 4, 0, 0)
    before = (ring.state(), ring.slot_block.copy(), ring.slot_pos.copy())
    with pytest.raises(ValueError):
        ring.write(np.zeros((11, 1, 2)), np.zeros((11, 1, 2)), 11, 0, 0)
    with pytest.raises(RingStateError):
        ring.write(np.zeros((3, 1, 2)), np.zeros((3, 1, 2)), 3, 0, 0)   # n != n_cur
    with pytest.raises(RingStateError):
        ring.write(z, z, 4, 1, 0)   # different position
    with pytest.raises(RingStateError):
        ring.advance(3)
    assert ring.state() == before[0]
    assert np.array_equal(ring.slot_block, before[1]) and np.array_equal(ring.slot_pos, before[2])
    ring.advance(4)
    with pytest.raises(RingStateError):
        ring.advance(4)   # nothing current


def test_wrap_and_eviction_slots():
    N = 96
    ring = Ring(N, 1, 2, "f32", 0.0)
    z = np.zeros((32, 1, 2))
    for b in range(3):
        ring.write(z, z, 32, 32 * b, b)
        ring.advance(32)
    assert ring.head == 0 and ring.n_hist == 96
    ring.write(z, z, 32, 96, 3)
    assert ring.n_hist == 64
    assert np.array_equal(ring.slot_block, np.repeat([3, 1, 2], 32))
    assert np.array_equal(ring.slot_pos[:32], np.arange(96, 128))
    # a write that wraps: head at 80, 32 tokens -> slots 80..95, 0..15
    ring2 = Ring(N, 1, 2, "f32", 0.0, first_slot=80)
    ring2.write(z, z, 32, 0, 0)
    assert np.array_equal(np.nonzero(ring2.slot_block == 0)[0], np.r_[0:16, 80:96])
    assert np.array_equal(ring2.slot_pos[80:96], np.arange(16))
    assert np.array_equal(ring2.slot_pos[0:16], np.arange(16, 32))


def test_anchor_slots_by_hand():
    """Anchor of 3 slots in a 10-slot ring, chunks of 3 tokens (chunk b has
    positions 3b..3b+2): slots 0..2 keep chunk 0, the sliding part 3..9
    wraps back to slot 3.  Expected contents derived by hand:
    chunk 1 -> 3,4,5; chunk 2 -> 6,7,8; chunk 3 -> 9,3,4; chunk 4 -> 5,6,7;
    chunk 5 -> 8,9,3."""
    N, A, n = 10, 3, 3
    ring = Ring(N, 1, 2, "f32", 0.0, n_anchor=A)
    z = np.zeros((n, 1, 2))
    heads = []
    for b in range(6):
        ring.write(z, z, n, 3 * b, b)
        ring.advance(n)
        heads.append(ring.head)
    assert heads == [3, 6, 9, 5, 8, 4]
    assert ring.n_hist == 10
    assert ring.slot_block.tolist() == [0, 0, 0, 5, 3, 4, 4, 4, 5, 5]
    assert ring.slot_pos.tolist() == [0, 1, 2, 17, 11, 12, 13, 14, 15, 16]
    # the next write evicts the two oldest sliding tokens (slots 4, 5), never the anchor
    ring.write(z[:2], z[:2], 2, 18, 6)
    assert ring.write_slots(2).tolist() == [4, 5] and ring.n_hist == 8
    assert ring.slot_block.tolist() == [0, 0, 0, 5, 6, 6, 4, 4, 5, 5]


def test_anchor_filled_by_a_straddling_chunk():
    """Anchor of 4 slots, chunks of 3: chunk 1 puts one token in the anchor
    and two in the sliding part; the wrap then returns to slot 4."""
    N, A, n = 10, 4, 3
    ring = Ring(N, 1, 2, "f32", 0.0, n_anchor=A)
    z = np.zeros((n, 1, 2))
    for b in range(4):
        ring.write(z, z, n, 3 * b, b)
        ring.advance(n)
    assert ring.head == 6
    assert ring.slot_block.tolist() == [0, 0, 0, 1, 3, 3, 2, 2, 2, 3]
    assert ring.slot_pos.tolist() == [0, 1, 2, 3, 10, 11, 6, 7, 8, 9]


def test_anchor_keeps_first_chunk_over_a_long_take():
    """The pages' shape: 5788 slots, chunks of 757 tokens, the first chunk
    pinned.  After every chunk the anchor still holds chunk 0 (positions
    0..756) and the sliding part holds the most recent 5031 tokens."""
    N, n = 5788, 757
    A = n
    ring = Ring(N, 1, 2, "f32", 0.0, n_anchor=A)
    z = np.zeros((n, 1, 2))
    for T in range(1, 30):
        ring.write(z, z, n, n * (T - 1), T - 1)
        ring.advance(n)
        assert np.all(ring.slot_block[:A] == 0)
        assert np.array_equal(ring.slot_pos[:A], np.arange(A))
        total = n * T
        recent = np.arange(max(A, total - (N - A)), total)  # token index = position
        held = np.sort(ring.slot_pos[A:][ring.slot_block[A:] != -1])
        assert np.array_equal(held, recent)
        assert ring.n_hist == min(total, N)


def test_anchor_argument_checks():
    with pytest.raises(ValueError):
        Ring(10, 1, 2, "f32", 0.0, n_anchor=10)
    with pytest.raises(ValueError):
        Ring(10, 1, 2, "f32", 0.0, n_anchor=-1)
    with pytest.raises(ValueError):
        Ring(10, 1, 2, "f32", 0.0, first_slot=2, n_anchor=3)
    ring = Ring(10, 1, 2, "f32", 0.0, n_anchor=3)
    with pytest.raises(ValueError):   # a chunk must fit the sliding part
        ring.write(np.zeros((8, 1, 2)), np.zeros((8, 1, 2)), 8, 0, 0)
    assert ring.state() == (0, 0, 0, 0, 0, 0)


@pytest.mark.parametrize("kv", ["fp8", "bf16", "f32"])
def test_write_stores_rotated_values(kv):
    rng = np.random.default_rng(5)
    N, H, d, n = 40, 3, 64, 17
    ring = Ring(N, H, d, kv, 10000.0, first_slot=30)
    k = rng.standard_normal((n, H, d))
    v = rng.standard_normal((n, H, d))
    ring.write(k, v, n, 500, 2)
    slots = (30 + np.arange(n)) % N
    k_exact = rope(k, (500 + np.arange(n))[:, None], 10000.0).transpose(1, 0, 2)
    v_exact = v.transpose(1, 0, 2)
    kc, vc = ring.k_values()[:, slots], ring.v_values()[:, slots]
    if kv == "fp8":
        ks = ring.k_scale[:, slots].astype(np.float64)[..., None]
        vs = ring.v_scale[:, slots].astype(np.float64)[..., None]
        # half of the largest code step (32, between 416 and 448) times the scale
        assert np.all(np.abs(kc - k_exact) <= 16 * ks + 1e-15)
        assert np.all(np.abs(vc - v_exact) <= 16 * vs + 1e-15)
        assert np.array_equal(ring.v_scale[:, slots], (np.max(np.abs(v_exact), -1) / 448).astype(np.float32))
    elif kv == "bf16":
        assert np.all(np.abs(kc - k_exact) <= np.abs(k_exact) * 2.0 ** -8)
        assert np.array_equal(vc, round_bf16(v_exact))
    else:
        assert np.array_equal(kc, k_exact.astype(np.float32).astype(np.float64))
    untouched = np.setdiff1d(np.arange(N), slots)
    assert np.all(ring.slot_block[untouched] == -1)


def test_round_bf16_against_float32_path():
    # For float32 inputs, bf16 rounding of the value equals the bit-level
    # round-to-nearest-even on the upper 16 bits.
    rng = np.random.default_rng(6)
    x = rng.standard_normal(100_000).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    want = r.astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.array_equal(round_bf16(x.astype(np.float64)), want)


def test_rerotate_equals_reencode_f32():
    rng = np.random.default_rng(8)
    N, H, d, n = 64, 2, 128, 50
    k = rng.standard_normal((n, H, d))
    a = Ring(N, H, d, "f32", 10000.0, first_slot=20)
    b = Ring(N, H, d, "f32", 10000.0, first_slot=20)
    a.write(k, k, n, 5031, 1)
    a.rerotate(-3000)
    b.write(k, k, n, 2031, 1)
    assert np.array_equal(a.slot_pos, b.slot_pos) and a.cur_pos0 == 2031
    ka, kb = a.k_values(), b.k_values()
    # two float32 roundings apart at most; a rotation moves rounding error
    # between the two members of a pair, so the bound uses the pair norm
    pn = np.sqrt(kb[..., 0::2] ** 2 + kb[..., 1::2] ** 2).repeat(2, axis=-1)
    assert np.all(np.abs(ka - kb) <= 4 * pn * 2.0 ** -24)


def test_rerotate_fp8_within_two_steps_of_reencode():
    rng = np.random.default_rng(9)
    N, H, d, n = 200, 4, 128, 150
    k = rng.standard_normal((n, H, d))
    a = Ring(N, H, d, "fp8", 10000.0, first_slot=120)
    b = Ring(N, H, d, "fp8", 10000.0, first_slot=120)
    a.write(k, k, n, 4000, 0)
    a.rerotate(-3000)
    b.write(k, k, n, 1000, 0)
    valid = a.slot_block != -1
    ka, kb = a.k_values()[:, valid], b.k_values()[:, valid]
    s = np.maximum(a.k_scale[:, valid], b.k_scale[:, valid]).astype(np.float64)[..., None]
    # each quantisation is off by at most half the top code step (16 * scale)
    assert np.all(np.abs(ka - kb) <= 3 * 16 * s * np.sqrt(2))
    # and a wrong angle would be far outside that: rotate by +3000 instead
    c = Ring(N, H, d, "fp8", 10000.0, first_slot=120)
    c.write(k, k, n, 4000, 0)
    c.rerotate(+3000)
    assert np.max(np.abs(c.k_values()[:, valid] - kb)) > 20 * np.max(s)
    # V and empty slots untouched
    assert np.array_equal(a.v, b.v)
    assert np.all(a.k[:, ~valid] == 0)
