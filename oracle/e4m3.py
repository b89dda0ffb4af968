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
and sign symmetry.
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
