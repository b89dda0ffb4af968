"""Pins for the oracle's QK-RMSNorm + split-half RoPE (CPU only)."""

import numpy as np
import pytest

from oracle import rmsnorm_rope_ref
from oracle.brute import rope_brute


def _x(seed, T=3, H=2, D=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, H, D)).astype(np.float16)


@pytest.mark.parametrize("pos", [0, 1, 8191])
@pytest.mark.parametrize("D", [64, 128])
def test_matches_mpmath_brute_force(pos, D):
    rng = np.random.default_rng(pos + D)
    x = rng.standard_normal((1, 2, D)).astype(np.float16)
    gamma = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    got = rmsnorm_rope_ref(x, gamma, np.array([pos]), 1e-6, 1e6)
    for h in range(2):
        want = np.array([float(v) for v in rope_brute(x[0, h], gamma, pos, 1e-6, 1e6)])
        # the float64 angle pos*f_i carries a relative error of ~1e-16, i.e.
        # ~1e-12 rad at pos = 8191: that is the float64 evaluation's own bound
        np.testing.assert_allclose(got[0, h], want, rtol=0, atol=5e-12)


def test_rms_of_output_with_unit_gamma():
    x = _x(1)
    eps = 1e-6
    y = rmsnorm_rope_ref(x, np.ones(16), np.array([0, 5, 77]), eps, 1e6)
    xf = x.astype(np.float64)
    ms = np.mean(xf ** 2, axis=-1)
    np.testing.assert_allclose(np.mean(y ** 2, axis=-1), ms / (ms + eps), rtol=1e-13)


def test_position_zero_is_plain_rmsnorm():
    x = _x(2)
    g = np.linspace(0.5, 1.5, 16)
    y = rmsnorm_rope_ref(x, g, np.zeros(3, dtype=int), 1e-6, 1e6)
    xf = x.astype(np.float64)
    want = xf / np.sqrt(np.mean(xf ** 2, axis=-1, keepdims=True) + 1e-6) * g
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-15)


def test_rotation_keeps_each_pair_norm():
    x = _x(3)
    g = np.ones(16)
    y0 = rmsnorm_rope_ref(x, g, np.zeros(3, dtype=int), 1e-6, 1e4)
    y = rmsnorm_rope_ref(x, g, np.array([3, 100, 4000]), 1e-6, 1e4)
    n0 = y0[..., :8] ** 2 + y0[..., 8:] ** 2
    n = y[..., :8] ** 2 + y[..., 8:] ** 2
    np.testing.assert_allclose(n, n0, rtol=1e-13)


def test_dot_product_depends_on_relative_position_only():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 32)).astype(np.float16)
    k = rng.standard_normal((1, 1, 32)).astype(np.float16)
    g = np.ones(32)

    def dot(m, n):
        a = rmsnorm_rope_ref(q, g, np.array([m]), 1e-6, 1e4)[0, 0]
        b = rmsnorm_rope_ref(k, g, np.array([n]), 1e-6, 1e4)[0, 0]
        return float(a @ b)

    assert abs(dot(10, 3) - dot(107, 100)) < 1e-11
    assert abs(dot(5, 5) - dot(0, 0)) < 1e-12
    assert abs(dot(10, 3) - dot(3, 10)) > 1e-6   # but not symmetric in sign of m-n


def test_first_pair_rotates_by_position_radians():
    """Element pair (0, D/2) has frequency theta^0 = 1: angle = pos."""
    x = np.zeros((1, 1, 8), dtype=np.float16)
    x[0, 0, 0] = 1.0
    pos = 3
    y = rmsnorm_rope_ref(x, np.ones(8), np.array([pos]), 0.0, 1e6)
    r = np.sqrt(8.0)          # RMS normalisation of a one-hot vector
    assert abs(y[0, 0, 0] - r * np.cos(pos)) < 1e-14
    assert abs(y[0, 0, 4] - r * np.sin(pos)) < 1e-14
