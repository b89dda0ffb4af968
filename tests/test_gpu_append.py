"""GPU parity of paged_kv_append (plain and Qwen3-fused) against the oracle.

Plain scatter: the whole pools must be bitwise equal to the oracle's
scatter (written rows and untouched bytes alike).  Fused: v and every
untouched byte bitwise; q' and k' within one fp16 ulp of the oracle's
once-rounded fp64 values (the kernel evaluates in fp32 with an fp64 angle).
Then append -> decode equals the oracle run on the oracle's appended pools.
"""

import numpy as np
import pytest
import torch

from oracle import append_ref, attn_ref, fused_append_ref
from paged_kv_cache_208_amd import _lib

from helpers import TOL_F16, batch, max_abs, run_decode, sample_seqs, to_device

pytestmark = pytest.mark.gpu


def _u16(x):
    return np.ascontiguousarray(x).view(np.uint16)


def _append(g, fused, cfg=None):
    kw = {}
    if fused:
        kw = dict(q=g["q"], gamma_q=g["gamma_q"], gamma_k=g["gamma_k"],
                  context_lens=g["context_lens"], eps=cfg.eps, rope_theta=cfg.theta)
    _lib.paged_kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["slot_mapping"],
                         **kw)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,kw", [("c2", dict(B=7, len_lo=1, len_hi=300, mbs=19)),
                                     ("c1", dict())])
def test_plain_append_is_bitwise(name, kw):
    cfg, d = batch(name, **kw)
    if d["k_new"] is None:   # c1 draws no new rows: make some
        rng = np.random.default_rng(3)
        d = dict(d, k_new=rng.standard_normal((cfg.B, cfg.Hkv, cfg.D)).astype(np.float16),
                 v_new=rng.standard_normal((cfg.B, cfg.Hkv, cfg.D)).astype(np.float16))
    slots = d["slot_mapping"].copy()
    slots[1] = -1                      # a skipped token
    d = dict(d, slot_mapping=slots)
    g = to_device(d)
    _append(g, False)
    kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], slots)
    assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
    assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))


def test_append_then_decode_matches_oracle():
    cfg, d = batch("c2", B=6, len_lo=1, len_hi=600, mbs=38)
    g = to_device(d)
    _append(g, False)
    kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], d["slot_mapping"])
    out = run_decode(cfg, g)
    ref = attn_ref(d["q"], kp, vp, d["block_tables"], d["context_lens"], cfg.scale)
    assert max_abs(out, ref) <= TOL_F16


def _check_fused(cfg, d, g, seqs=None):
    q2, kp, vp, qx, kx = fused_append_ref(d["q"], d["k_new"], d["v_new"], d["k_pool"],
                                          d["v_pool"], d["slot_mapping"], d["context_lens"],
                                          d["gamma_q"], d["gamma_k"], cfg.eps, cfg.theta)
    gq = g["q"].cpu().numpy()
    gk = g["k_pool"].cpu().numpy()
    gv = g["v_pool"].cpu().numpy()
    # q' within one fp16 ulp of the exact value's rounding
    dq = np.abs(gq.astype(np.float64) - q2.astype(np.float64))
    ulp = np.spacing(np.maximum(np.abs(q2), np.abs(gq)).astype(np.float16)).astype(np.float64)
    assert np.all(dq <= ulp), f"q' off by {np.max(dq / ulp):.2f} ulp"
    # v and every untouched byte bitwise; k' rows within one ulp
    assert np.array_equal(_u16(gv), _u16(vp))
    written = np.zeros(gk.shape[:3], dtype=bool)   # [NB, Hkv, BS]
    for s in d["slot_mapping"]:
        if s >= 0:
            written[s // 16, :, s % 16] = True
    assert np.array_equal(_u16(gk)[~written], _u16(kp)[~written])
    dk = np.abs(gk[written].astype(np.float64) - kp[written].astype(np.float64))
    ulpk = np.spacing(np.maximum(np.abs(kp[written]), np.abs(gk[written])).astype(np.float16))
    assert np.all(dk <= ulpk.astype(np.float64))
    return q2, kp, vp


@pytest.mark.parametrize("D", [64, 128])
def test_fused_append_small(D):
    kw = dict(B=9, len_lo=1, len_hi=8192, mbs=512)
    if D == 64:
        kw.update(D=64, Hq=8, Hkv=2)
    cfg, d = batch("c4", **kw)
    g = to_device(d)
    _append(g, True, cfg)
    q2, kp, vp = _check_fused(cfg, d, g)
    out = run_decode(cfg, g)
    ref = attn_ref(q2, kp, vp, d["block_tables"], d["context_lens"], cfg.scale)
    assert max_abs(out, ref) <= TOL_F16


def test_fused_append_positions_up_to_8191():
    """RoPE angles up to pos 8191 (theta 1e6): the fp64 angle keeps q'/k'
    within one ulp of the oracle at every position."""
    cfg, d = batch("c4", B=16, len_lo=8000, len_hi=8192, mbs=512)
    lens = d["context_lens"].copy()
    lens[0] = 8192                                    # pos 8191
    lens[1] = 1                                       # pos 0: plain RMSNorm
    tab = d["block_tables"]
    slots = np.array([int(tab[b, (lens[b] - 1) // 16]) * 16 + (lens[b] - 1) % 16
                      for b in range(cfg.B)], dtype=np.int64)
    d = dict(d, context_lens=lens, slot_mapping=slots)
    g = to_device(d)
    _append(g, True, cfg)
    _check_fused(cfg, d, g)


def test_full_size_fused_append_decode():
    """Qwen3-8B-shaped B=256: fused append + partitioned decode + reduce in
    the bench's launch configuration; sampled sequences against the oracle."""
    cfg, d = batch("c4")
    g = to_device(d)
    _append(g, True, cfg)
    out = run_decode(cfg, g)
    o = out.cpu().double().numpy()
    assert np.all(np.isfinite(o))
    seqs = sample_seqs(cfg.B, 5, seed=2)
    q2, kp, vp, _, _ = fused_append_ref(d["q"][seqs], d["k_new"][seqs], d["v_new"][seqs],
                                        d["k_pool"], d["v_pool"], d["slot_mapping"][seqs],
                                        d["context_lens"][seqs], d["gamma_q"], d["gamma_k"],
                                        cfg.eps, cfg.theta)
    ref = attn_ref(q2, kp, vp, d["block_tables"][seqs], d["context_lens"][seqs], cfg.scale)
    err = float(np.max(np.abs(o[seqs] - ref)))
    print(f"c4 sampled {seqs} max_abs={err:.3e}", flush=True)
    assert err <= TOL_F16
