"""QKV projection feeding the cache write (oracle, float64).

Test infrastructure only (see ``oracle/__init__.py``).

Runway Characters (abstract) serves its 57B model with FP8 GEMMs and writes
each chunk's keys and values into the ring cache once, with RoPE and FP8
quantisation at write time.  The projection that produces them, read
plainly, with FP8 operands:

* the layer input x [n][C] (bfloat16 values) is quantised per token:
  scale = max|x_t| / 448 (float32), codes = round-to-nearest-even(x / scale)
  -- the same rule as every FP8 vector in the cache;
* the weights W [3 H d][C] are e4m3 codes with one float32 scale per output
  row (synthetic: there are no trained weights);
* [q | k | v] = dequant(x) . dequant(W)^T, exactly (float64 here); rows
  0..H d - 1 of W give q (head-major, d per head), then k, then v.
q is handed to the attention unrotated (rounded to bfloat16, the format the
attention takes); k and v go to the ring as any write: k rotated at its
position, then both quantised per (token, head).
"""
from __future__ import annotations

import numpy as np

from . import e4m3


def quantize_tokens(x: np.ndarray):
    """Per-token FP8 quantisation of x [n][C]: (codes uint8 [n][C], scales
    float32 [n])."""
    return e4m3.quantize(np.asarray(x, dtype=np.float64))


def qkv_project(x: np.ndarray, w_codes: np.ndarray, w_scale: np.ndarray, n_heads: int, head_dim: int):
    """x: float64 [n][C] (bfloat16 values); w_codes uint8 [3 H d][C];
    w_scale float32 [3 H d].  Returns (q, k, v), each float64 [n][H][d]."""
    n, C = x.shape
    HD = n_heads * head_dim
    if w_codes.shape != (3 * HD, C) or w_scale.shape != (3 * HD,):
        raise ValueError("w must be [3 H d][C] with one scale per row")
    xc, xs = quantize_tokens(x)
    xd = e4m3.dequantize(xc, xs)                 # [n][C]
    wd = e4m3.dequantize(w_codes, w_scale)       # [3 H d][C]
    out = xd @ wd.T                              # [n][3 H d], float64
    q, k, v = (out[:, i * HD:(i + 1) * HD].reshape(n, n_heads, head_dim) for i in range(3))
    return q, k, v
