"""E4M3 KV on the GPU: precision that does not depend on the data's scale,
every code decoded exactly, and blocks whose scale is zero.

The FP8 KV cache ("Roadmap: vLLM-style serving features for TornadoVM
batched decode", Sampling / logits) stores value = e4m3(code) * scale per
(block, kv head).  The kernels apply the V scale's power of two inside the
code conversion and its mantissa to the softmax weights, so neither fp16
operand of the P.V product leaves fp16's normal range; the error relative to
the output's magnitude must then stay the same from tiny to large data.
Every path that reads E4M3 tiles is covered: paged_attn_decode single pass
and partitioned (+ paged_attn_reduce), paged_decode_step balanced and with
fixed partitions.
"""

import numpy as np
import pytest
import torch

from oracle import attn_ref, e4m3_table
from paged_kv_cache_208_amd import _lib, synth

from helpers import TOL_E4M3, batch, dev, to_device

pytestmark = pytest.mark.gpu

# max-abs error / max |output| (oracle on the same E4M3 bytes, fp64): the
# softmax weights are rounded to fp16 once (relative 2^-11) and everything
# else is exact or fp32, so the bound is about four fp16 ulps of the output
# scale whatever the data scale
REL_TOL_E4M3 = 2e-3

PATHS = ["decode", "decode_ps512", "step_balanced", "step_ps512"]


def run_path(path, cfg, g, q=None, lens=None, tables=None):
    q = g["q"] if q is None else q
    lens = g["context_lens"] if lens is None else lens
    tables = g["block_tables"] if tables is None else tables
    B, Hq, D = q.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    sc = dict(k_scale=g["k_scale"], v_scale=g["v_scale"])
    if path.startswith("decode"):
        ps = 512 if path.endswith("ps512") else 0
        _lib.decode_step(out, q, g["k_pool"], g["v_pool"], tables, lens, cfg.scale,
                         partition_size=ps, **sc)
    else:
        ps = 512 if path.endswith("ps512") else 0
        P = _lib.max_partitions_for(tables.shape[1], ps) if ps else 16
        ws = _lib.alloc_step_workspace(B, Hq, cfg.Hkv, D, P)
        _lib.paged_decode_step(out, q, g["k_pool"], g["v_pool"], tables, lens, cfg.scale,
                               partition_size=ps, workspace=ws, **sc)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("sigma", [1e-3, 1e-1, 1.0, 100.0])
@pytest.mark.parametrize("path", PATHS)
def test_e4m3_error_relative_to_the_output_scale(sigma, path):
    cfg, d = batch("c5", B=4, len_lo=300, len_hi=1500, mbs=94, kv_sigma=sigma)
    g = to_device(d)
    out = run_path(path, cfg, g)
    ref = attn_ref(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                   cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"])
    o = out.cpu().double().numpy()
    assert np.all(np.isfinite(o))
    rel = float(np.max(np.abs(o - ref)) / np.max(np.abs(ref)))
    print(f"sigma={sigma:g} {path}: max|out|={np.max(np.abs(ref)):.3e} "
          f"max-abs/max|out|={rel:.3e}", flush=True)
    assert rel <= REL_TOL_E4M3
    if sigma == 1.0:
        assert float(np.max(np.abs(o - ref))) <= TOL_E4M3


def _all_codes_batch(v_scale):
    """Two one-token sequences (g = 8, D = 128): V row 0 of sequence 0 holds
    codes 0x00..0x7F, of sequence 1 codes 0x80..0xFF (the two NaN codes
    replaced by zeros of their sign), K row 0 is 1.0 everywhere; every other
    row and block is NaN."""
    Hq, Hkv, D, NB = 8, 1, 128, 4
    kp = np.full((NB, Hkv, 16, D), 0x7F, dtype=np.uint8)
    vp = np.full((NB, Hkv, 16, D), 0x7F, dtype=np.uint8)
    codes = np.arange(256, dtype=np.int32)
    codes[0x7F], codes[0xFF] = 0x00, 0x80
    for b, blk in enumerate((1, 2)):
        kp[blk, 0, 0] = 0x38
        vp[blk, 0, 0] = codes[128 * b:128 * (b + 1)]
    ks = np.full((NB, Hkv), np.nan, dtype=np.float32)
    vs = np.full((NB, Hkv), np.nan, dtype=np.float32)
    ks[1:3] = 1.0
    vs[1:3] = v_scale
    tables = np.array([[1, 3], [2, 3]], dtype=np.int32)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, Hq, D)).astype(np.float16)
    return dict(q=q, k_pool=kp, v_pool=vp, k_scale=ks, v_scale=vs, block_tables=tables,
                context_lens=np.array([1, 1], dtype=np.int32)), codes


@pytest.mark.parametrize("v_scale", [1.0, 2.0 ** -10, 0.75, 3.0])
@pytest.mark.parametrize("path", PATHS)
def test_every_finite_code_decodes_exactly(v_scale, path):
    """With one token the softmax weight is exactly 1, so every output
    element is that token's V value: all 254 finite codes times the scale,
    rounded once to fp16, which is exact for these scales."""
    d, codes = _all_codes_batch(v_scale)
    cfg = synth.CONFIGS["c5"].replace(B=2, Hq=8, Hkv=1, mbs=2)
    g = to_device(d)
    out = run_path(path, cfg, g)
    want = (e4m3_table()[codes].reshape(2, 128) * v_scale)
    assert np.all(np.isfinite(want))
    want16 = want.astype(np.float16)
    assert np.array_equal(want16.astype(np.float64), want)       # exact in fp16
    got = out.cpu().numpy()                                          # [2, 8, 128]
    for b in range(2):
        for h in range(8):
            # value equality (the sum 0 + 1 * (-0) of the P.V product is +0,
            # so code 0x80 comes back as +0); every other element bitwise
            assert np.array_equal(got[b, h].astype(np.float64), want16[b].astype(np.float64)), \
                (b, h, np.nonzero(got[b, h].astype(np.float64) != want16[b].astype(np.float64)))
            nz = want16[b] != 0
            assert np.array_equal(got[b, h][nz].view(np.uint16), want16[b][nz].view(np.uint16))


@pytest.mark.parametrize("path", PATHS)
def test_zero_k_scale_in_a_partly_filled_block(path):
    """A block whose K rows are all zero has K scale 0 (the E4M3 append
    writes exactly that while a block holds only zero rows).  Its logits are
    0, never -inf * 0: the output stays finite and equals the oracle's."""
    cfg, d = batch("c5", B=4, len_lo=20, len_hi=900, mbs=57)
    kp, ks = d["k_pool"].copy(), d["k_scale"].copy()
    for b, L in enumerate(d["context_lens"]):
        L = int(L)
        last = int(d["block_tables"][b, (L - 1) // 16])
        kp[last, :, :(L - 1) % 16 + 1] = 0x00
        ks[last] = 0.0
        mid = int(d["block_tables"][b, 0])     # and a full (or first) block
        kp[mid, :, :min(16, L)] = 0x80
        ks[mid] = 0.0
    d2 = dict(d, k_pool=kp, k_scale=ks)
    g = to_device(d2)
    out = run_path(path, cfg, g)
    ref = attn_ref(d2["q"], kp, d2["v_pool"], d2["block_tables"], d2["context_lens"], cfg.scale,
                   k_scale=ks, v_scale=d2["v_scale"])
    o = out.cpu().double().numpy()
    assert np.all(np.isfinite(o))
    assert float(np.max(np.abs(o - ref))) <= TOL_E4M3
