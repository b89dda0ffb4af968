"""Roofline helpers for the decode measurement.

The ridge point of a roofline is peak compute divided by peak memory
bandwidth ("Distributed LLM Inference Serving Platform", section 6.2 and the
Lab 3 roofline calculator in section 11).  Kernels whose FLOP per byte sits
below it are bandwidth bound.
"""

# MI355X published peaks (dense, no sparsity)
HBM_GBPS = 8000.0
MFMA_F16_TFLOPS = 2500.0
VALU_F32_TFLOPS = 157.3
VALU_F64_TFLOPS = 78.6


def ridge_point(peak_tflops: float, peak_bw_gbps: float) -> float:
    """FLOP per byte at which compute and bandwidth limits meet."""
    return (peak_tflops * 1e12) / (peak_bw_gbps * 1e9)


def decode_flops(context_tokens: int, Hq: int, D: int) -> int:
    """FLOPs of one decode step's attention: q.k and p.v per token and q head,
    each a D-long multiply-add (2 FLOP per element)."""
    return 4 * int(context_tokens) * Hq * D
