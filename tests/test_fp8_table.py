"""Pins for the oracle's E4M3 decode table (CPU only).

The table is built from the format's closed form in oracle/e4m3.py; here it
is checked code by code against torch's independent float8_e4m3fn decoder,
and against landmark values of the OCP E4M3 definition worked out by hand
from the bit fields (tests/golden/e4m3_landmarks.json).
"""

import json
import math
import os

import numpy as np
import torch

from oracle.e4m3 import e4m3_decode, e4m3_table


def test_all_codes_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = e4m3_table()
    for c in range(256):
        if math.isnan(ref[c]):
            assert math.isnan(tab[c]), c
        else:
            assert tab[c] == ref[c], (c, tab[c], ref[c])
            assert math.copysign(1, tab[c]) == math.copysign(1, ref[c]), c


def test_landmarks_of_the_format():
    t = e4m3_table()
    assert t[0x00] == 0.0 and math.copysign(1, t[0x80]) == -1.0
    assert t[0x01] == 2.0 ** -9                 # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert t[0x08] == 2.0 ** -6                 # smallest normal
    assert t[0x38] == 1.0                       # exponent field 7 = bias
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert np.nanmax(np.abs(t)) == 448.0
    assert np.sum(np.isnan(t)) == 2


def test_hand_worked_landmark_codes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "e4m3_landmarks.json")))
    t = e4m3_table()
    assert len(g["codes"]) >= 12
    for c in g["codes"]:
        code = int(c["code"], 16)
        if c["value"] == "nan":
            assert math.isnan(t[code]), c
        else:
            assert t[code] == c["value"], c
            assert math.copysign(1, t[code]) == math.copysign(1, c["value"]), c


def test_positive_codes_are_monotone_and_sign_symmetric():
    t = e4m3_table()
    pos = t[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)
    np.testing.assert_array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def test_decode_requires_uint8():
    import pytest
    with pytest.raises(TypeError):
        e4m3_decode(np.zeros(3, dtype=np.int32))
