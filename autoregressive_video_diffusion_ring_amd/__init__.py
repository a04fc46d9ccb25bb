"""Ring-cache chunk attention on AMD Instinct MI355X (gfx950).

Python binding of the C ABI in ``include/rc.h`` (librc.so).  PyTorch is used
only for device memory and streams; every step of the path runs in the HIP
kernels behind the C ABI.  The entry points keep the C names:

    rc_ring_init, rc_cache_write, rc_cache_rerotate, rc_chunk_attention,
    rc_ring_advance, rc_attention_workspace_bytes, rc_debug_visibility,
    rc_key_mass, rc_key_mass_slots, rc_key_mass_workspace_bytes,
    rc_cache_write_scored, rc_cache_write_scored_workspace_bytes,
    rc_chunk_attention_ex, rc_qkv_project_write, rc_qkv_workspace_bytes,
    rc_set_attention_precision, rc_chunk_attention_noalloc, rc_attention_noalloc_limit

and ``Ring`` owns a ring's device buffers (torch tensors) and its rc_ring
struct.  See include/rc.h for the meaning of every argument.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (DTYPES, RC_BF16, RC_F32, RC_FP8_E4M3, RC_MASK_BLOCK_CAUSAL, RC_MASK_SAME_BLOCK,
                   RC_PRECISION_AUTO, RC_PRECISION_ONE_TERM, RC_PRECISION_TWO_TERM, RcError, RcRing, check, lib)

__all__ = [
    "Ring", "RcError", "RcRing", "rc_ring_init", "rc_cache_write", "rc_cache_rerotate",
    "rc_chunk_attention", "rc_ring_advance", "rc_attention_workspace_bytes", "rc_debug_visibility",
    "rc_debug_tile_classes", "rc_debug_tile_classes_bytes",
    "rc_chunk_attention_noalloc", "rc_attention_noalloc_limit",
    "rc_ring_sizes", "rc_ring_v_ld", "rc_key_mass", "rc_key_mass_slots", "rc_key_mass_workspace_bytes",
    "rc_cache_write_scored",
    "rc_cache_write_scored_workspace_bytes", "rc_chunk_attention_ex", "RC_MASK_BLOCK_CAUSAL", "RC_MASK_SAME_BLOCK",
    "rc_qkv_project_write", "rc_qkv_workspace_bytes", "rc_set_attention_precision", "RC_PRECISION_AUTO",
    "RC_PRECISION_TWO_TERM", "RC_PRECISION_ONE_TERM",
]


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _input_dtype(kv_dtype: int) -> torch.dtype:
    return torch.float32 if kv_dtype == RC_F32 else torch.bfloat16


def _check_tensor(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


# ------------------------------------------------------------------ C names
def rc_ring_v_ld(n_slots: int) -> int:
    return lib().rc_ring_v_ld(n_slots)


def rc_ring_sizes(n_slots: int, n_heads: int, head_dim: int, kv_dtype: int) -> list[int]:
    out = (ctypes.c_size_t * 6)()
    check(lib().rc_ring_sizes(n_slots, n_heads, head_dim, kv_dtype, out))
    return list(out)


def rc_ring_init(ring: RcRing, first_slot: int, stream=None) -> None:
    check(lib().rc_ring_init(ctypes.byref(ring), first_slot, _stream(stream)))


def rc_cache_write(ring: RcRing, k_new, v_new, n_new: int, pos0: int, block_id: int, stream=None) -> None:
    check(lib().rc_cache_write(ctypes.byref(ring), _ptr(k_new), _ptr(v_new), n_new, pos0, block_id,
                               _stream(stream)))


def rc_cache_rerotate(ring: RcRing, delta: int, stream=None) -> None:
    check(lib().rc_cache_rerotate(ctypes.byref(ring), delta, _stream(stream)))


def rc_chunk_attention(ring: RcRing, q, n_q: int, q_pos0: int, q_block0: int, q_block_len: int,
                       cache_bias: float, softmax_scale: float, out, lse=None, workspace=None,
                       workspace_bytes: int = 0, stream=None) -> None:
    check(lib().rc_chunk_attention(ctypes.byref(ring), _ptr(q), n_q, q_pos0, q_block0, q_block_len,
                                   float(cache_bias), float(softmax_scale), _ptr(out), _ptr(lse),
                                   _ptr(workspace), workspace_bytes, _stream(stream)))


def rc_chunk_attention_ex(ring: RcRing, q, n_q: int, q_pos0: int, q_block, q_block0: int, q_block_len: int,
                          mask: int, cache_bias: float, softmax_scale: float, out, lse=None, workspace=None,
                          workspace_bytes: int = 0, stream=None) -> None:
    check(lib().rc_chunk_attention_ex(ctypes.byref(ring), _ptr(q), n_q, q_pos0, _ptr(q_block), q_block0,
                                      q_block_len, mask, float(cache_bias), float(softmax_scale), _ptr(out),
                                      _ptr(lse), _ptr(workspace), workspace_bytes, _stream(stream)))


def rc_qkv_project_write(ring: RcRing, x, n: int, C: int, w, w_scale, pos0: int, block_id: int, q_out, workspace,
                         workspace_bytes: int, stream=None) -> None:
    check(lib().rc_qkv_project_write(ctypes.byref(ring), _ptr(x), n, C, _ptr(w), _ptr(w_scale), pos0, block_id,
                                     _ptr(q_out), _ptr(workspace), workspace_bytes, _stream(stream)))


def rc_qkv_workspace_bytes(n: int, C: int) -> int:
    return lib().rc_qkv_workspace_bytes(n, C)


def rc_set_attention_precision(mode: int) -> None:
    check(lib().rc_set_attention_precision(mode))


def rc_attention_workspace_bytes(ring: RcRing, n_q: int) -> int:
    return lib().rc_attention_workspace_bytes(ctypes.byref(ring), n_q)


def rc_chunk_attention_noalloc(ring: RcRing, q, n_q: int, q_pos0: int, q_block0: int, q_block_len: int,
                               cache_bias: float, softmax_scale: float, out, lse=None, stream=None) -> None:
    check(lib().rc_chunk_attention_noalloc(ctypes.byref(ring), _ptr(q), n_q, q_pos0, q_block0, q_block_len,
                                           float(cache_bias), float(softmax_scale), _ptr(out), _ptr(lse),
                                           _stream(stream)))


def rc_attention_noalloc_limit() -> int:
    return lib().rc_attention_noalloc_limit()


def rc_ring_advance(ring: RcRing, n: int) -> None:
    check(lib().rc_ring_advance(ctypes.byref(ring), n))


def rc_key_mass(ring: RcRing, q, n_q: int, q_pos0: int, q_block0: int, q_block_len: int, cache_bias: float,
                softmax_scale: float, lse, mass, workspace, workspace_bytes: int, stream=None) -> None:
    check(lib().rc_key_mass(ctypes.byref(ring), _ptr(q), n_q, q_pos0, q_block0, q_block_len, float(cache_bias),
                            float(softmax_scale), _ptr(lse), _ptr(mass), _ptr(workspace), workspace_bytes,
                            _stream(stream)))


def rc_key_mass_slots(ring: RcRing, q, n_q: int, q_pos0: int, q_block0: int, q_block_len: int, cache_bias: float,
                      softmax_scale: float, lse, ranges, mass, workspace, workspace_bytes: int, stream=None) -> None:
    """ranges: a sequence of (lo, hi) slot ranges (host ints)."""
    flat = [int(v) for pair in ranges for v in pair]
    arr = (ctypes.c_int32 * max(len(flat), 1))(*flat)
    check(lib().rc_key_mass_slots(ctypes.byref(ring), _ptr(q), n_q, q_pos0, q_block0, q_block_len,
                                  float(cache_bias), float(softmax_scale), _ptr(lse), arr, len(flat) // 2,
                                  _ptr(mass), _ptr(workspace), workspace_bytes, _stream(stream)))


def rc_key_mass_workspace_bytes(ring: RcRing, n_q: int) -> int:
    return lib().rc_key_mass_workspace_bytes(ctypes.byref(ring), n_q)


def rc_cache_write_scored(ring: RcRing, k_new, v_new, n_new: int, pos0: int, block_id: int, key_score,
                          diversity: float, workspace, workspace_bytes: int, stream=None) -> None:
    check(lib().rc_cache_write_scored(ctypes.byref(ring), _ptr(k_new), _ptr(v_new), n_new, pos0, block_id,
                                      _ptr(key_score), float(diversity), _ptr(workspace), workspace_bytes,
                                      _stream(stream)))


def rc_cache_write_scored_workspace_bytes(ring: RcRing, n_new: int) -> int:
    return lib().rc_cache_write_scored_workspace_bytes(ctypes.byref(ring), n_new)


def rc_debug_visibility(ring: RcRing, n_q: int, q_block0: int, q_block_len: int, mask, stream=None) -> None:
    check(lib().rc_debug_visibility(ctypes.byref(ring), n_q, q_block0, q_block_len, _ptr(mask),
                                    _stream(stream)))


def rc_debug_tile_classes_bytes(ring: RcRing, n_q: int) -> int:
    return lib().rc_debug_tile_classes_bytes(ctypes.byref(ring), n_q)


def rc_debug_tile_classes(ring: RcRing, n_q: int, q_block0: int, q_block_len: int, mask: int, cache_bias: float,
                          classes, classes_bytes: int, stream=None) -> None:
    check(lib().rc_debug_tile_classes(ctypes.byref(ring), n_q, q_block0, q_block_len, mask, float(cache_bias),
                                      _ptr(classes), classes_bytes, _stream(stream)))


# ------------------------------------------------------------------ owner
class Ring:
    """One layer's ring cache: device buffers as torch tensors plus the
    rc_ring struct the C ABI maintains."""

    def __init__(self, n_slots: int, n_heads: int, head_dim: int, kv_dtype: str = "fp8",
                 rope_base: float = 10000.0, first_slot: int = 0, n_anchor: int = 0,
                 n_memory: int = 0, device="cuda", stream=None):
        self.kv = DTYPES[kv_dtype]
        self.kv_name = kv_dtype
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        sizes = rc_ring_sizes(n_slots, n_heads, head_dim, self.kv)
        self.buffers = [torch.empty(max(s, 16), dtype=torch.uint8, device=self.device) if s else None
                        for s in sizes]
        s = self.struct = RcRing()
        s.n_slots, s.n_heads, s.head_dim, s.kv_dtype = n_slots, n_heads, head_dim, self.kv
        s.rope_base = rope_base
        s.v_ld = rc_ring_v_ld(n_slots)
        s.n_anchor = n_anchor
        s.n_memory = n_memory
        s.k, s.v, s.k_scale, s.v_scale, s.slot_pos, s.slot_block = (_ptr(b) for b in self.buffers)
        rc_ring_init(s, first_slot, stream)

    # geometry
    N = property(lambda self: self.struct.n_slots)
    H = property(lambda self: self.struct.n_heads)
    d = property(lambda self: self.struct.head_dim)
    v_ld = property(lambda self: self.struct.v_ld)
    n_anchor = property(lambda self: self.struct.n_anchor)
    n_memory = property(lambda self: self.struct.n_memory)
    input_dtype = property(lambda self: _input_dtype(self.kv))

    def state(self) -> tuple[int, int, int, int, int, int]:
        s = self.struct
        return (s.head, s.n_hist, s.n_cur, s.cur_pos0, s.cur_block, s.n_mem)

    def write(self, k_new, v_new, pos0: int, block_id: int, stream=None) -> None:
        n = k_new.shape[0]
        shape = (n, self.H, self.d)
        _check_tensor(k_new, "k_new", self.input_dtype, shape, self.device)
        _check_tensor(v_new, "v_new", self.input_dtype, shape, self.device)
        rc_cache_write(self.struct, k_new, v_new, n, pos0, block_id, stream)

    def write_scored(self, k_new, v_new, pos0: int, block_id: int, key_score, diversity: float = 1.0,
                     workspace=None, stream=None) -> None:
        n = k_new.shape[0]
        shape = (n, self.H, self.d)
        _check_tensor(k_new, "k_new", self.input_dtype, shape, self.device)
        _check_tensor(v_new, "v_new", self.input_dtype, shape, self.device)
        _check_tensor(key_score, "key_score", torch.float32, (self.H, self.v_ld), self.device)
        if workspace is None:
            need = rc_cache_write_scored_workspace_bytes(self.struct, n)
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device) if need else None
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc_cache_write_scored(self.struct, k_new, v_new, n, pos0, block_id, key_score, diversity, workspace,
                              ws_bytes, stream)

    def key_mass(self, q, q_pos0: int, q_block0: int, q_block_len: int | None, cache_bias: float, lse,
                 mass=None, softmax_scale: float = 0.0, workspace=None, stream=None, ranges=None):
        """Accumulate the attention mass of q's rows into mass [H][v_ld]
        (a new zero tensor when None); lse is rc_chunk_attention's output.
        ranges: optional (lo, hi) slot ranges; only their slots are scored."""
        n_q = q.shape[0]
        _check_tensor(q, "q", self.input_dtype, (n_q, self.H, self.d), self.device)
        _check_tensor(lse, "lse", torch.float32, (self.H, n_q), self.device)
        if mass is None:
            mass = torch.zeros((self.H, self.v_ld), dtype=torch.float32, device=self.device)
        _check_tensor(mass, "mass", torch.float32, (self.H, self.v_ld), self.device)
        if workspace is None:
            need = rc_key_mass_workspace_bytes(self.struct, n_q)
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device)
        ws_bytes = workspace.numel() * workspace.element_size()
        if ranges is None:
            rc_key_mass(self.struct, q, n_q, q_pos0, q_block0, q_block_len or n_q, cache_bias, softmax_scale, lse,
                        mass, workspace, ws_bytes, stream)
        else:
            rc_key_mass_slots(self.struct, q, n_q, q_pos0, q_block0, q_block_len or n_q, cache_bias, softmax_scale,
                              lse, ranges, mass, workspace, ws_bytes, stream)
        return mass

    def project_write(self, x, w, w_scale, pos0: int, block_id: int, q_out=None, workspace=None, stream=None):
        """Fused QKV projection + cache write of the tokens of x [n][C] (bf16);
        w: uint8 e4m3 codes [3 H d][C], w_scale float32 [3 H d].  Returns q
        [n][H][d] (bf16, not rotated)."""
        n, C = x.shape
        _check_tensor(x, "x", torch.bfloat16, (n, C), self.device)
        _check_tensor(w, "w", torch.uint8, (3 * self.H * self.d, C), self.device)
        _check_tensor(w_scale, "w_scale", torch.float32, (3 * self.H * self.d,), self.device)
        if q_out is None:
            q_out = torch.empty((n, self.H, self.d), dtype=torch.bfloat16, device=self.device)
        _check_tensor(q_out, "q_out", torch.bfloat16, (n, self.H, self.d), self.device)
        if workspace is None:
            workspace = torch.empty(max(rc_qkv_workspace_bytes(n, C), 16), dtype=torch.uint8, device=self.device)
        rc_qkv_project_write(self.struct, x, n, C, w, w_scale, pos0, block_id, q_out, workspace,
                             workspace.numel() * workspace.element_size(), stream)
        return q_out

    def rerotate(self, delta: int, stream=None) -> None:
        rc_cache_rerotate(self.struct, delta, stream)

    def advance(self, n: int) -> None:
        rc_ring_advance(self.struct, n)

    def workspace_bytes(self, n_q: int) -> int:
        return rc_attention_workspace_bytes(self.struct, n_q)

    def attention(self, q, q_pos0: int, q_block0: int, q_block_len: int | None = None,
                  cache_bias: float = 0.0, softmax_scale: float = 0.0, out=None, lse=None,
                  workspace=None, stream=None, q_block=None, same_block: bool = False):
        """q_block: optional int32 [n_q] device tensor of per-query blocks;
        same_block: the text cross-attention mask (slot block == query block)."""
        n_q = q.shape[0]
        shape = (n_q, self.H, self.d)
        _check_tensor(q, "q", self.input_dtype, shape, self.device)
        if out is None:
            out = torch.empty(shape, dtype=self.input_dtype, device=self.device)
        _check_tensor(out, "out", self.input_dtype, shape, self.device)
        if lse is not None:
            _check_tensor(lse, "lse", torch.float32, (self.H, n_q), self.device)
        ws_bytes = 0
        if workspace is None:
            need = self.workspace_bytes(n_q)
            if need:
                workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        if workspace is not None:
            ws_bytes = workspace.numel() * workspace.element_size()
        if q_block is None and not same_block:
            rc_chunk_attention(self.struct, q, n_q, q_pos0, q_block0, q_block_len or n_q, cache_bias,
                               softmax_scale, out, lse, workspace, ws_bytes, stream)
        else:
            if q_block is not None:
                _check_tensor(q_block, "q_block", torch.int32, (n_q,), self.device)
            rc_chunk_attention_ex(self.struct, q, n_q, q_pos0, q_block, q_block0, q_block_len or n_q,
                                  RC_MASK_SAME_BLOCK if same_block else RC_MASK_BLOCK_CAUSAL, cache_bias,
                                  softmax_scale, out, lse, workspace, ws_bytes, stream)
        return out

    def visibility(self, n_q: int, q_block0: int, q_block_len: int, stream=None):
        mask = torch.empty((n_q, self.N), dtype=torch.uint8, device=self.device)
        rc_debug_visibility(self.struct, n_q, q_block0, q_block_len, mask, stream)
        return mask

    def tile_classes(self, n_q: int, q_block0: int, q_block_len: int, cache_bias: float = 0.0,
                     same_block: bool = False, stream=None):
        """The FP8 attention kernel's half-tile classes, uint8 [ceil(n_q/32)][ceil(N/128)][2]
        (bits: 1 vis, 2 fast, 4 hist)."""
        shape = ((n_q + 31) // 32, (self.N + 127) // 128, 2)
        classes = torch.empty(shape, dtype=torch.uint8, device=self.device)
        rc_debug_tile_classes(self.struct, n_q, q_block0, q_block_len,
                              RC_MASK_SAME_BLOCK if same_block else RC_MASK_BLOCK_CAUSAL, cache_bias, classes,
                              classes.numel(), stream)
        return classes

    # ---- read-back in the logical layout [H][N][d] (copies, for checking)
    def _view(self, i, dtype, shape):
        b = self.buffers[i]
        n = 1
        for x in shape:
            n *= x
        return b.view(dtype)[:n].view(*shape)

    def _elem_dtype(self):
        return {RC_F32: torch.float32, RC_BF16: torch.bfloat16, RC_FP8_E4M3: torch.uint8}[self.kv]

    def k_raw(self):
        return self._view(0, self._elem_dtype(), (self.H, self.v_ld, self.d))[:, :self.N].clone()

    def v_raw(self):
        vt = self._view(1, self._elem_dtype(), (self.H, self.d, self.v_ld))
        return vt[:, :, :self.N].transpose(1, 2).contiguous()

    def k_scale(self):
        if self.kv != RC_FP8_E4M3:
            return None
        return self._view(2, torch.float32, (self.H, self.v_ld))[:, :self.N].clone()

    def v_scale(self):
        if self.kv != RC_FP8_E4M3:
            return None
        return self._view(3, torch.float32, (self.H, self.v_ld))[:, :self.N].clone()

    def slot_pos(self):
        return self._view(4, torch.int32, (self.v_ld,))[:self.N].clone()

    def slot_block(self):
        return self._view(5, torch.int32, (self.v_ld,))[:self.N].clone()
