"""Rotary position encoding (oracle, float64).

Test infrastructure only (see ``oracle/__init__.py``).

The pages apply RoPE to each key once, when it is written, and to the
queries (Runway Characters, abstract); they do not give its form.  The
reading taken is the original rotary encoding on adjacent pairs:

    theta_i = base^(-2i/d),  i = 0 .. d/2-1
    phi     = pos * theta_i
    x'[2i]   = x[2i] cos(phi) - x[2i+1] sin(phi)
    x'[2i+1] = x[2i] sin(phi) + x[2i+1] cos(phi)

with 1-D token positions.  Because rotations compose, R(p + delta) =
R(delta) R(p): a cached key is moved to a new position by rotating it by
delta alone, which is the delta rotation applied on a position reset.
"""
from __future__ import annotations

import numpy as np


def thetas(head_dim: int, base: float) -> np.ndarray:
    """Frequencies theta_i = base^(-2i/d) for i < d/2 (float64)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the last axis of x (length d, even) by positions ``pos``.

    ``pos`` broadcasts against x.shape[:-1] (e.g. shape [n, 1] for x of shape
    [n, H, d]).  base == 0 means no rotation (the identity)."""
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    d = x.shape[-1]
    th = thetas(d, base)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * th  # [..., d/2]
    c, s = np.cos(phi), np.sin(phi)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, phi.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
