"""The circular (ring) KV cache: write, delta re-rotation, advance (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Runway Characters (abstract) moves the whole-cache work of every attention
call to write time: a ring cache, RoPE and FP8 quantisation applied once per
write, and a delta rotation of the cached keys when positions reset.  The
bookkeeping below is the plainest reading of "ring cache":

* N slots per layer.  ``head`` is the next slot to write.
* A write of n tokens (1 <= n <= N) goes to slots (head + i) mod N, i < n.
  History occupies the n_hist slots just before ``head``; the write covers
  the oldest of them when n_hist + n > N, so after it
  n_hist = min(n_hist, N - n).
* Every denoising pass of the same chunk writes again (same n, positions and
  block) into the same slots until the chunk is committed by ``advance``.
* ``advance(n)``: head = (head + n) mod N, n_hist += n, n_cur = 0.
* Each slot records its token position and block id; block -1 marks a slot
  never written.
* ``rerotate(delta)``: every written slot's key is dequantised, rotated by
  delta and quantised again; its position moves by delta; V is untouched.

Anchor + sliding window ("Why Live Video Generation Still Struggles With
Timing", transcript: a streaming editor keeps the first chunk as a permanent
anchor beside a window of recent history; StreamLTX project page, "Why a long
take does not slow down": an anchor next to a FIFO of recent blocks).
Plainest reading, with A = n_anchor pinned slots (0 = the plain ring):

* the first A tokens ever written fill slots 0..A-1 and stay there;
* every later token goes to the sliding part, slots A..N-1, as a ring of
  N - A slots: token k of the stream (k >= A; the passes of one chunk
  rewrite the same tokens) lands in slot A + (k - A) mod (N - A).
In head terms: a write of n tokens goes to head + i while that is below N
and wraps to A + (head + i - N); a chunk must fit the sliding part
(n <= N - A), so a write never covers an anchor slot once they are filled.
An anchored ring starts at slot 0.  n_hist keeps its meaning (committed
tokens in the cache, anchor included) and its update rules.

Content memory (StreamLTX project page, "Why a long take does not slow
down": besides the anchor and the FIFO of recent blocks, a content memory
whose keys each layer scores, keeping a top-M budget).  With M = n_memory
slots the memory is slots E..N-1, E = N - M, and the sliding part shrinks to
A..E-1 (writes wrap from E to A; a chunk holds at most E - A tokens; n_hist
counts the anchor and sliding tokens, up to E).  A plain write lets the
tokens it overwrites go.  A scored write (``write_scored``) first lets them
compete with the memory's tokens for its M slots: see ``oracle.memory`` for
the score and the selection.  n_mem counts the occupied memory slots.

Storage per layer, logical layout [H][N][d]:
* fp8:  K and V as e4m3fn codes plus float32 scales [H][N];
* bf16: K and V rounded to bfloat16 (nearest, ties to even);
* f32:  K and V rounded to float32.
"""
from __future__ import annotations

import numpy as np

from . import e4m3
from .rope import rope


class RingStateError(ValueError):
    """A call that the ring's host state does not allow."""


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits; magnitudes here stay far inside its
    normal range, which the assertion checks."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    nz = x != 0
    assert np.all(np.abs(x[nz]) > 2.0 ** -120), "bf16 subnormal range not modelled"
    q = np.rint(m * 256.0)  # rint rounds half to even
    return np.ldexp(q / 256.0, e)


def _round_store(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "bf16":
        return round_bf16(x)
    if kv_dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    raise ValueError(kv_dtype)


class Ring:
    """One layer's ring cache plus its host state."""

    def __init__(self, n_slots: int, n_heads: int, head_dim: int, kv_dtype: str,
                 rope_base: float, first_slot: int = 0, n_anchor: int = 0,
                 n_memory: int = 0):
        if kv_dtype not in ("fp8", "bf16", "f32"):
            raise ValueError(kv_dtype)
        if n_slots < 1 or n_heads < 1 or head_dim < 2 or head_dim % 2:
            raise ValueError("bad ring shape")
        if not 0 <= first_slot < n_slots:
            raise ValueError("first_slot out of range")
        if n_anchor < 0 or n_memory < 0 or n_anchor + n_memory >= n_slots:
            raise ValueError("need n_anchor, n_memory >= 0 and n_anchor + n_memory < N")
        if n_anchor > 0 and first_slot != 0:
            raise ValueError("an anchored ring starts at slot 0")
        if first_slot >= n_slots - n_memory:
            raise ValueError("first_slot must lie before the memory slots")
        self.N, self.H, self.d = n_slots, n_heads, head_dim
        self.A = n_anchor
        self.M = n_memory
        self.E = n_slots - n_memory  # end of the sliding part
        self.kv_dtype = kv_dtype
        self.rope_base = float(rope_base)
        shape = (n_heads, n_slots, head_dim)
        if kv_dtype == "fp8":
            self.k = np.zeros(shape, dtype=np.uint8)
            self.v = np.zeros(shape, dtype=np.uint8)
            self.k_scale = np.zeros((n_heads, n_slots), dtype=np.float32)
            self.v_scale = np.zeros((n_heads, n_slots), dtype=np.float32)
        else:
            self.k = np.zeros(shape, dtype=np.float64)
            self.v = np.zeros(shape, dtype=np.float64)
            self.k_scale = self.v_scale = None
        self.slot_pos = np.zeros(n_slots, dtype=np.int64)
        self.slot_block = np.full(n_slots, -1, dtype=np.int64)
        self.head = first_slot
        self.n_hist = 0
        self.n_cur = 0
        self.cur_pos0 = 0
        self.cur_block = 0
        self.n_mem = 0

    # ----------------------------------------------------------- accessors
    def state(self) -> tuple[int, int, int, int, int, int]:
        return (self.head, self.n_hist, self.n_cur, self.cur_pos0, self.cur_block, self.n_mem)

    def k_values(self) -> np.ndarray:
        """Cached keys as float64 [H][N][d] (dequantised for fp8)."""
        if self.kv_dtype == "fp8":
            return e4m3.dequantize(self.k, self.k_scale)
        return self.k.copy()

    def v_values(self) -> np.ndarray:
        """Cached values as float64 [H][N][d] (dequantised for fp8)."""
        if self.kv_dtype == "fp8":
            return e4m3.dequantize(self.v, self.v_scale)
        return self.v.copy()

    def _step(self, i):
        """Slot i places after head, wrapping from the end of the sliding
        part (E; N without a memory) back to its first slot (A; 0 without an
        anchor)."""
        s = self.head + np.asarray(i)
        return np.where(s < self.E, s, s - self.E + self.A)

    def write_slots(self, n: int) -> np.ndarray:
        """Slots a write of n tokens goes to: head + i, wrapped into A..E-1
        ((head + i) mod N for the plain ring)."""
        return self._step(np.arange(n))

    # ------------------------------------------------------------- writes
    def _encode_into(self, dst, dst_scale, slots, x_hnd):
        """Store x [H][n][d] (float64) into slots of dst."""
        if self.kv_dtype == "fp8":
            codes, scale = e4m3.quantize(x_hnd)
            dst[:, slots, :] = codes
            dst_scale[:, slots] = scale
        else:
            dst[:, slots, :] = _round_store(x_hnd, self.kv_dtype)

    def write(self, k_new: np.ndarray, v_new: np.ndarray, n: int, pos0: int,
              block_id: int) -> None:
        """Write n new tokens; k_new and v_new are float64 [n][H][d]."""
        if not 1 <= n <= self.E - self.A:
            raise ValueError("n_new must be in 1..N - n_anchor - n_memory")
        if block_id < 0:
            raise ValueError("block_id must be >= 0")
        k_new = np.asarray(k_new, dtype=np.float64)
        v_new = np.asarray(v_new, dtype=np.float64)
        if k_new.shape != (n, self.H, self.d) or v_new.shape != (n, self.H, self.d):
            raise ValueError("k_new/v_new must be [n][H][d]")
        if self.n_cur > 0 and (n != self.n_cur or pos0 != self.cur_pos0
                               or block_id != self.cur_block):
            raise RingStateError("a rewrite must repeat the current chunk's n, pos0, block")
        if self.n_cur == 0:
            self.n_hist = min(self.n_hist, self.E - n)
        slots = self.write_slots(n)
        positions = pos0 + np.arange(n)
        k_rot = rope(k_new, positions[:, None], self.rope_base)  # [n][H][d]
        self._encode_into(self.k, self.k_scale, slots, k_rot.transpose(1, 0, 2))
        self._encode_into(self.v, self.v_scale, slots, v_new.transpose(1, 0, 2))
        self.slot_pos[slots] = positions
        self.slot_block[slots] = block_id
        self.n_cur, self.cur_pos0, self.cur_block = n, pos0, block_id

    def write_scored(self, k_new: np.ndarray, v_new: np.ndarray, n: int, pos0: int,
                     block_id: int, key_score: np.ndarray, diversity: float) -> None:
        """A write whose evicted history tokens first compete with the
        memory's tokens for the M memory slots (first pass of a chunk only;
        later passes and rings without a memory write as ``write``).

        key_score: float32 values [H][N] (e.g. attention mass per head and
        slot); diversity: gamma in (0, 1]."""
        from .memory import select_memory  # the selection rule lives there

        if not 0.0 < diversity <= 1.0:
            raise ValueError("diversity must be in (0, 1]")
        if not 1 <= n <= self.E - self.A:
            raise ValueError("n_new must be in 1..N - n_anchor - n_memory")
        if block_id < 0:
            raise ValueError("block_id must be >= 0")
        if np.shape(k_new) != (n, self.H, self.d) or np.shape(v_new) != (n, self.H, self.d):
            raise ValueError("k_new/v_new must be [n][H][d]")
        if self.M > 0 and self.n_cur == 0:
            evicted = [int(s) for s in self.write_slots(n) if self.slot_block[s] != -1]
            held = [s for s in range(self.E, self.N) if self.slot_block[s] != -1]
            keep = set(select_memory(held + evicted, self.slot_block, key_score, self.M, diversity))
            incoming = sorted(s for s in keep if s < self.E)          # winners from the sliding part
            free = [s for s in range(self.E, self.N) if s not in keep]  # empty or a loser's
            for src, dst in zip(incoming, free):                      # both in ascending order
                self.k[:, dst] = self.k[:, src]
                self.v[:, dst] = self.v[:, src]
                if self.kv_dtype == "fp8":
                    self.k_scale[:, dst] = self.k_scale[:, src]
                    self.v_scale[:, dst] = self.v_scale[:, src]
                self.slot_pos[dst] = self.slot_pos[src]
                self.slot_block[dst] = self.slot_block[src]
            self.n_mem = len(keep)
        self.write(k_new, v_new, n, pos0, block_id)

    def rerotate(self, delta: int) -> None:
        """Rotate every written slot's key by delta; positions move by delta."""
        valid = np.nonzero(self.slot_block != -1)[0]
        if valid.size:
            k = self.k_values()[:, valid, :]  # [H][nv][d]
            k_rot = rope(k, np.full((1, valid.size), delta), self.rope_base)
            self._encode_into(self.k, self.k_scale, valid, k_rot)
            self.slot_pos[valid] += delta
        if self.n_cur > 0:
            self.cur_pos0 += delta

    def advance(self, n: int) -> None:
        """Commit the current chunk of n tokens as history."""
        if self.n_cur == 0 or n != self.n_cur:
            raise RingStateError("advance(n) needs n == n_cur > 0")
        self.head = int(self._step(n))
        self.n_hist = min(self.n_hist + n, self.E)
        self.n_cur = 0

    # ---------------------------------------------------------- transport
    @classmethod
    def from_arrays(cls, *, kv_dtype, rope_base, k, v, k_scale, v_scale, slot_pos,
                    slot_block, state=(0, 0, 0, 0, 0, 0), n_anchor=0, n_memory=0):
        """Build a ring from given cache contents (logical layout [H][N][d])."""
        H, N, d = k.shape
        r = cls(N, H, d, kv_dtype, rope_base, n_anchor=n_anchor, n_memory=n_memory)
        if kv_dtype == "fp8":
            r.k = np.array(k, dtype=np.uint8)
            r.v = np.array(v, dtype=np.uint8)
            r.k_scale = np.array(k_scale, dtype=np.float32)
            r.v_scale = np.array(v_scale, dtype=np.float32)
        else:
            r.k = np.array(k, dtype=np.float64)
            r.v = np.array(v, dtype=np.float64)
        r.slot_pos = np.array(slot_pos, dtype=np.int64)
        r.slot_block = np.array(slot_block, dtype=np.int64)
        st = tuple(int(x) for x in state) + (0,) * (6 - len(state))
        r.head, r.n_hist, r.n_cur, r.cur_pos0, r.cur_block, r.n_mem = st
        return r
