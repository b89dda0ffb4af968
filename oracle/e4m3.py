"""FP8 E4M3 decode table for the quantized-KV read path (oracle side).

The pages list a quantized (Q8/FP8) KV cache as a planned item
("Roadmap: vLLM-style serving features for TornadoVM batched decode",
Sampling / logits) without fixing a format.  The reading adopted is the OCP
8-bit floating point E4M3 format (the "FN" variant): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, no infinities, and a single NaN pattern
per sign (exponent and mantissa all ones).  Largest finite value 448.

Every code is decoded from that closed form here, in Python integers and
exact float64 arithmetic (every E4M3 value is a dyadic rational that float64
holds exactly).

Pins (tests/test_fp8_table.py): all 256 codes against torch.float8_e4m3fn
bit for bit, hand-written values of the format's landmark codes
(tests/golden/e4m3_landmarks.json), monotonicity of the positive codes,
and sign symmetry.  The encoder (e4m3_encode) is pinned against torch's
float32 -> float8_e4m3fn cast (round to nearest even) on every float16
value in range and on random float32 values and exact midpoints, and by
encode(decode(c)) == c for every finite code.
"""

import math

import numpy as np

_TABLE = None


def _decode_code(code: int) -> float:
    """Value of one E4M3 byte, straight from the format definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        # subnormal: no implicit leading one, exponent fixed at 1 - bias = -6
        return sign * math.ldexp(man / 8.0, -6)
    return sign * math.ldexp(1.0 + man / 8.0, exp - 7)


def e4m3_table() -> np.ndarray:
    """float64[256]: value of every E4M3 code (NaN for the two NaN codes)."""
    global _TABLE
    if _TABLE is None:
        _TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)
        _TABLE.setflags(write=False)
    return _TABLE


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to float64 through the table."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("e4m3 codes must be uint8")
    return e4m3_table()[codes]


E4M3_MAX = 448.0


def e4m3_encode(values) -> np.ndarray:
    """Nearest E4M3 code of each float32 value, ties to the even code
    (round-to-nearest-even on the 3-bit mantissa), magnitudes above 448
    clamped to 448, the sign kept (also for values that round to zero).

    Written from the format: the finite non-negative codes 0..126 are
    ordered by value, so the nearest code is found by comparing the value
    with its two neighbours in the table, exactly in float64 (every float32
    and every E4M3 value is exact there).  NaN input is not handled.
    """
    v = np.asarray(values, dtype=np.float32).astype(np.float64)
    mags = e4m3_table()[:127]                      # codes 0x00..0x7E, ascending
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(mags, a, side="left")     # first code with value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a >= mags[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = np.signbit(v)
    return np.where(sign, code | 0x80, code).astype(np.uint8)
