"""Pins for the oracle's QKV projection (oracle/projection.py).

* Brute force: explicit loops over (token, output row, input column) with
  the codes decoded one by one, on a small case.
* Closed form: weights that are unit rows (code 0x38 = 1.0 at one column,
  scale 2^-k) pick single quantised input columns, scaled.
* The token quantisation is the cache's own per-vector rule (all codes of a
  token's absmax element are +-448, the scale is fl32(max/448)).
"""
import numpy as np

from oracle import e4m3
from oracle.projection import qkv_project, quantize_tokens
from synthetic_inputs import normal_bf16


def test_brute_force_small():
    rng = np.random.default_rng(0)
    n, C, H, d = 3, 16, 2, 4
    _, x = normal_bf16(rng, (n, C))
    codes = rng.integers(0, 0x7E, size=(3 * H * d, C), dtype=np.uint8) | (
        rng.integers(0, 2, size=(3 * H * d, C), dtype=np.uint8) << 7)
    ws = rng.uniform(0.001, 0.01, size=3 * H * d).astype(np.float32)
    q, k, v = qkv_project(x, codes, ws, H, d)
    xc, xs = quantize_tokens(x)
    table = [e4m3.decode(c) for c in range(256)]
    for t in range(n):
        for r in range(3 * H * d):
            acc = 0.0
            for c in range(C):
                acc += (table[xc[t, c]] * float(xs[t])) * (table[codes[r, c]] * float(ws[r]))
            which, rem = divmod(r, H * d)
            h, j = divmod(rem, d)
            got = (q, k, v)[which][t, h, j]
            assert abs(got - acc) <= 1e-12 * max(1.0, abs(acc))


def test_unit_rows_pick_columns():
    rng = np.random.default_rng(1)
    n, C, H, d = 5, 64, 2, 8
    _, x = normal_bf16(rng, (n, C))
    cols = rng.integers(0, C, size=3 * H * d)
    codes = np.zeros((3 * H * d, C), dtype=np.uint8)
    codes[np.arange(3 * H * d), cols] = 0x38            # 1.0 in e4m3
    ws = (2.0 ** -rng.integers(0, 6, size=3 * H * d)).astype(np.float32)
    q, k, v = qkv_project(x, codes, ws, H, d)
    xd = e4m3.dequantize(*quantize_tokens(x))
    expect = xd[:, cols] * ws.astype(np.float64)[None, :]
    got = np.concatenate([a.reshape(n, H * d) for a in (q, k, v)], axis=1)
    assert np.array_equal(got, expect)


def test_token_quantisation_rule():
    rng = np.random.default_rng(2)
    _, x = normal_bf16(rng, (4, 128))
    codes, scale = quantize_tokens(x)
    for t in range(4):
        a = np.max(np.abs(x[t]))
        assert scale[t] == np.float32(np.float32(a) / np.float32(448.0))
        assert set(codes[t][np.abs(x[t]) == a]) <= {0x7E, 0xFE}
