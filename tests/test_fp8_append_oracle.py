"""Pins of the E4M3 encoder and of the E4M3 append oracle
(oracle/e4m3.py e4m3_encode, oracle/fp8_append.py append_e4m3_ref)."""

import numpy as np
import pytest
import torch

from oracle import append_e4m3_ref, e4m3_encode, e4m3_table

F32 = np.float32


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_encoder_matches_torch_on_every_float16_in_range():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h) & (np.abs(h.astype(np.float64)) <= 448)]
    assert np.array_equal(e4m3_encode(h.astype(F32)), _torch_codes(h.astype(F32)))


def test_encoder_matches_torch_at_midpoints_and_random_values():
    t = e4m3_table()[:127]
    mid = ((t[:-1] + t[1:]) / 2).astype(F32)          # exact in float32
    for x in (mid, -mid, np.nextafter(mid, F32(1e9)), np.nextafter(mid, F32(-1e9))):
        assert np.array_equal(e4m3_encode(x), _torch_codes(x))
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * rng.choice([1e-4, 1e-2, 1, 40, 400], 100000)).astype(F32)
    x = x[np.abs(x) <= 448]
    assert np.array_equal(e4m3_encode(x), _torch_codes(x))


def test_encoder_round_trips_every_finite_code_and_clamps():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_table()[codes].astype(F32)), codes)
    assert e4m3_encode(F32(1e6)) == 0x7E and e4m3_encode(F32(-1e6)) == 0xFE
    assert e4m3_encode(F32(-0.0)) == 0x80 and e4m3_encode(F32(1e-9)) == 0x00


def _half_spacing(v):
    """Half the E4M3 spacing around |v| (in units of the scaled value)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))


def _one_block(rows, Hkv=2, D=32, stale=None, bs=16):
    """Append `rows` ([n][Hkv][D] fp16) one per call into block 3 of a pool
    of `bs`-token blocks."""
    NB = 6
    kp = np.zeros((NB, Hkv, bs, D), dtype=np.uint8) if stale is None else stale.copy()
    vp = kp.copy()
    ks = np.full((NB, Hkv), 7.0, dtype=F32)    # stale scales: a new block ignores them
    vs = ks.copy()
    hist = []
    for r, x in enumerate(rows):
        kp, vp, ks, vs = append_e4m3_ref(kp, vp, ks, vs, x[None], x[None],
                                         np.array([3 * bs + r], dtype=np.int64), block_size=bs)
        hist.append((kp.copy(), ks.copy()))
    return hist


@pytest.mark.parametrize("bs", [16, 32])
def test_scale_tracks_running_amax_and_values_stay_within_rounding(bs):
    """bs = 32: the same policy over a 32-token block ("Distributed LLM
    Inference Serving Platform", section 12), slots block * 32 + row."""
    rng = np.random.default_rng(3)
    mags = [0.5, 2.0, 1.0, 40.0, 3.0, 300.0, 0.01, 300.0, 1e-3, 7.0, 7.0, 90.0, 1.0, 2.0, 0.0, 500.0]
    if bs == 32:
        mags = mags + [0.2, 600.0, 1.0, 1e-2, 5.0, 5.0, 0.0, 700.0, 3.0, 2.0, 1.0, 40.0, 8.0, 9.0,
                       0.5, 1.0]
    rows = [(rng.standard_normal((2, 32)) * m).astype(np.float16) for m in mags]
    hist = _one_block(rows, bs=bs)
    tab = e4m3_table()
    prev_codes = prev_scale = None
    for r, (kp, ks) in enumerate(hist):
        amax_rows = np.max(np.abs(np.stack(rows[: r + 1]).astype(F32)), axis=(0, 2))  # [Hkv]
        assert np.array_equal(ks[3], (amax_rows / F32(448)).astype(F32)), r
        # rows written before this one change only if the amax grew
        if prev_codes is not None:
            for h in range(2):
                if ks[3, h] == prev_scale[h]:
                    assert np.array_equal(kp[3, h, :r], prev_codes[h, :r])
        prev_codes, prev_scale = kp[3].copy(), ks[3].copy()
        # the newest row is one rounding from its exact value
        for h in range(2):
            x = rows[r][h].astype(np.float64)
            s = float(ks[3, h])
            got = tab[kp[3, h, r]] * s
            bound = _half_spacing(x / s) * s if s > 0 else 0 * x
            assert np.all(np.abs(got - x) <= bound * (1 + 1e-5) + 1e-30), (r, h)
    # every row at the end: one rounding per encoding it went through (its
    # own, plus one per later growth of the scale), each at most half a
    # spacing: 2^-4 of the value in the normal range, 2^-10 * s below it
    kp, ks = hist[-1]
    for h in range(2):
        s = float(ks[3, h])
        scales = [float(hs[3, h]) for _, hs in hist]
        for r in range(bs):
            k = sum(1 for j in range(r + 1, bs) if scales[j] != scales[j - 1])
            x = rows[r][h].astype(np.float64)
            got = tab[kp[3, h, r]] * s
            bound = (k + 1) * (2.0 ** -4 * np.abs(x) * 1.1 + 2.0 ** -10 * s)
            assert np.all(np.abs(got - x) <= bound), (r, h, k)


def test_equal_magnitudes_hit_the_largest_code_and_new_block_ignores_stale_bytes():
    stale = np.random.default_rng(4).integers(0, 126, (6, 1, 16, 16), dtype=np.uint8)
    x = np.full((1, 16), -3.0, dtype=np.float16)
    x[0, ::2] = 3.0
    kp, ks = _one_block([x.reshape(1, 16)], Hkv=1, D=16, stale=stale)[-1]
    assert ks[3, 0] == F32(3.0) / F32(448)
    assert set(kp[3, 0, 0].tolist()) == {0x7E, 0xFE}
    assert np.array_equal(kp[3, 0, 1:], stale[3, 0, 1:])     # other rows untouched
    others = [b for b in range(6) if b != 3]
    assert np.array_equal(kp[others], stale[others])


def test_zero_rows_and_skipped_slots():
    kp = np.zeros((2, 1, 16, 8), dtype=np.uint8)
    ks = np.zeros((2, 1), dtype=F32)
    z = np.zeros((1, 1, 8), dtype=np.float16)
    kp2, _, ks2, _ = append_e4m3_ref(kp, kp, ks, ks, z, z, np.array([16], dtype=np.int64))
    assert ks2[1, 0] == 0 and not kp2.any()
    kp3, _, ks3, _ = append_e4m3_ref(kp2, kp2, ks2, ks2, z + 1, z + 1, np.array([-1], dtype=np.int64))
    assert np.array_equal(kp3, kp2) and np.array_equal(ks3, ks2)
    one = np.full((1, 1, 8), 2.0, dtype=np.float16)
    kp4, _, ks4, _ = append_e4m3_ref(kp2, kp2, ks2, ks2, one, one, np.array([17], dtype=np.int64))
    assert ks4[1, 0] == F32(2.0) / F32(448) and np.all(kp4[1, 0, 0] == 0)
    assert np.all(kp4[1, 0, 1] == 0x7E)
