"""Pins for the oracle's RoPE (adjacent pairs, theta_i = base^(-2i/d)).

Pinned by: the identity at position 0, pair norms, composition
R(a)R(b) = R(a+b) (the property the delta rotation relies on), relative
position invariance of dot products, an independent complex-number
formulation with the angle read back by atan2, and closed-form frequencies
(tests/golden/rope_thetas.txt).
"""
import os

import numpy as np
import pytest

from oracle.rope import rope, thetas

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rope_thetas.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            d, i, t = line.split()
            rows.append((int(d), int(i), float(t)))
    return rows


@pytest.mark.parametrize("d,i,theta", _golden())
def test_theta_closed_forms(d, i, theta):
    assert thetas(d, 10000.0)[i] == pytest.approx(theta, rel=1e-14)


@pytest.mark.parametrize("d,i,theta", _golden())
def test_rotation_angle_read_back(d, i, theta):
    # rotate the unit vector e_{2i}; the pair (x'_{2i}, x'_{2i+1}) must sit at
    # angle pos * theta_i, measured independently with atan2.
    for pos in (1, 7, 100, 5787, -3000):
        x = np.zeros(d)
        x[2 * i] = 1.0
        y = rope(x, pos, 10000.0)
        ang = np.arctan2(y[2 * i + 1], y[2 * i])
        want = np.angle(np.exp(1j * pos * theta))
        assert abs(np.angle(np.exp(1j * (ang - want)))) < 1e-9
        others = np.delete(y, [2 * i, 2 * i + 1])
        assert np.all(others == 0)


def test_complex_formulation():
    rng = np.random.default_rng(1)
    d = 64
    x = rng.standard_normal((5, 3, d))
    pos = np.array([0, 3, 96, 5000, -17])
    y = rope(x, pos[:, None], 10000.0)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    th = np.array([10.0 ** (-8.0 * i / d) for i in range(d // 2)])
    zr = z * np.exp(1j * pos[:, None, None] * th)
    assert np.allclose(y[..., 0::2], zr.real, atol=1e-12)
    assert np.allclose(y[..., 1::2], zr.imag, atol=1e-12)


def test_identity_and_norms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 128))
    assert np.array_equal(rope(x, np.zeros((10,)), 10000.0), x)
    assert np.array_equal(rope(x, np.arange(10), 0.0), x)
    y = rope(x, np.arange(10) * 777, 10000.0)
    n0 = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    n1 = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-13)


def test_composition():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 128))
    for a, b in [(5031, -3000), (12, 13), (100000, 2345)]:
        assert np.allclose(rope(rope(x, a, 1e4), b, 1e4), rope(x, a + b, 1e4), atol=1e-9)


def test_relative_position_invariance():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    for p, r, delta in [(5031, 17, -3000), (100, 90, 5788), (0, 5787, 123456)]:
        a = rope(q, p + delta, 1e4) @ rope(k, r + delta, 1e4)
        b = rope(q, p, 1e4) @ rope(k, r, 1e4)
        assert abs(a - b) < 1e-9
