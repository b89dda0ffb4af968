"""Pins for the oracle's KV append and fused Qwen3 prologue (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import append_ref, fused_append_ref, rmsnorm_rope_ref


@pytest.mark.parametrize("fixture", ["append_scatter.json", "append_scatter_bs32.json"])
def test_scatter_matches_hand_written_fixture(golden_dir, fixture):
    g = json.load(open(os.path.join(golden_dir, fixture)))
    nb, hkv, bs, d = g["nb"], g["hkv"], g["block_size"], g["d"]
    k_pool = np.full((nb, hkv, bs, d), -7, dtype=np.float16)
    v_pool = np.full((nb, hkv, bs, d), -9, dtype=np.float16)
    k_new = np.array(g["k_new"], dtype=np.float16)
    v_new = -k_new
    kp, vp = append_ref(k_pool, v_pool, k_new, v_new, np.array(g["slot_mapping"]), bs)
    expect_k = k_pool.copy()
    expect_v = v_pool.copy()
    for w in g["expected_writes"]:
        expect_k[w["block"], :, w["row"], :] = k_new[w["token"]]
        expect_v[w["block"], :, w["row"], :] = v_new[w["token"]]
    np.testing.assert_array_equal(kp, expect_k)
    np.testing.assert_array_equal(vp, expect_v)
    # the skipped token (slot -1) wrote nothing: only the listed rows differ
    assert np.sum(np.any(kp != k_pool, axis=-1)) == len(g["expected_writes"]) * hkv
    # inputs are not modified
    assert np.all(k_pool == -7)


def test_fused_rounds_once_to_fp16_and_copies_v():
    rng = np.random.default_rng(0)
    T, Hq, Hkv, D = 3, 4, 2, 16
    q = rng.standard_normal((T, Hq, D)).astype(np.float16)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    pools = [np.zeros((4, Hkv, 16, D), dtype=np.float16) for _ in range(2)]
    lens = np.array([1, 20, 64], dtype=np.int32)
    slots = np.array([5, 16 + 3, 3 * 16 + 15], dtype=np.int64)
    gq = rng.uniform(0.8, 1.2, D).astype(np.float32)
    gk = rng.uniform(0.8, 1.2, D).astype(np.float32)
    q2, kp, vp, qx, kx = fused_append_ref(q, k, v, pools[0], pools[1], slots, lens,
                                          gq, gk, 1e-6, 1e6)
    np.testing.assert_array_equal(q2, rmsnorm_rope_ref(q, gq, lens - 1, 1e-6, 1e6).astype(np.float16))
    # once-rounded: the stored value is the float16 nearest the exact value
    err = np.abs(q2.astype(np.float64) - qx)
    ulp = np.spacing(np.abs(q2).astype(np.float16)).astype(np.float64)
    assert np.all(err <= 0.5 * ulp + 1e-300)
    np.testing.assert_array_equal(kp[0, :, 5], kx[0].astype(np.float16))
    np.testing.assert_array_equal(vp[1, :, 3], v[1])
    np.testing.assert_array_equal(vp[3, :, 15], v[2])


def test_numpy_float64_to_float16_is_round_to_nearest_even():
    """The oracle's only rounding step, checked against exact rational
    rounding on values around fp16 grid points and exact ties."""
    from fractions import Fraction
    rng = np.random.default_rng(1)
    grid = rng.standard_normal(2000).astype(np.float16).astype(np.float64)
    ups = np.nextafter(grid.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    ties = (grid + ups) / 2                           # exact midpoints
    near = ties + rng.uniform(-1, 1, ties.shape) * 1e-3 * (ups - grid)
    for x, lo, hi in zip(np.concatenate([ties, near]), np.tile(grid, 2), np.tile(ups, 2)):
        a, b = sorted([lo, hi])
        fx, fa, fb = Fraction(x), Fraction(a), Fraction(b)
        if fx - fa < fb - fx:
            want = a
        elif fx - fa > fb - fx:
            want = b
        else:   # tie: even mantissa
            want = a if (np.float16(a).view(np.uint16) & 1) == 0 else b
        assert np.float64(np.float16(x)) == want, (x, a, b)
