"""32-token blocks ("Distributed LLM Inference Serving Platform", section 12,
production readiness checklist: standardise on 16 or 32 tokens per physical
block): the balanced step, the appends and the copy on pools of
[NB][Hkv][32][D], against the oracle with block_size = 32."""

import numpy as np
import pytest
import torch

from oracle import (append_e4m3_ref, append_ref, attn_ref, copy_blocks_ref, fused_append_ref,
                    mq_attn_ref)
from paged_kv_cache_208_amd import _lib

from helpers import TOL_E4M3, TOL_F16, batch, dev, max_abs, to_device

pytestmark = pytest.mark.gpu
BS = 32


def _u16(x):
    return np.ascontiguousarray(x).view(np.uint16)


def _step(cfg, g, *, k_new=None, v_new=None, q=None, window=0, qknorm=False, nq=1):
    q = g["q"] if q is None else q
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float16, device="cuda")
    ws = _lib.alloc_step_workspace(cfg.B, cfg.Hq * nq, cfg.Hkv, cfg.D, 16)
    kw = {}
    if qknorm:
        kw = dict(gamma_q=g["gamma_q"], gamma_k=g["gamma_k"], eps=cfg.eps, rope_theta=cfg.theta)
    _lib.paged_decode_step(out, q, g["k_pool"], g["v_pool"], g["block_tables"], g["context_lens"],
                           cfg.scale, k_new=k_new, v_new=v_new, k_scale=g.get("k_scale"),
                           v_scale=g.get("v_scale"), partition_size=0, window=window,
                           workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[3]).item() == 0
    return out


@pytest.mark.parametrize("window", [0, 100])
def test_step_block32_append_attend(window):
    cfg, d = batch("c2", B=9, len_lo=1, len_hi=700, mbs=22, block_size=BS)
    g = to_device(d)
    out = _step(cfg, g, k_new=g["k_new"], v_new=g["v_new"], window=window)
    kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], d["slot_mapping"],
                        block_size=BS)
    assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
    assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))
    ref = attn_ref(d["q"], kp, vp, d["block_tables"], d["context_lens"], cfg.scale,
                   block_size=BS, window=window)
    assert max_abs(out, ref) <= TOL_F16


def test_step_block32_qknorm_and_e4m3():
    cfg, d = batch("c4", B=7, len_lo=1, len_hi=1000, mbs=32, block_size=BS)
    g = to_device(d)
    out = _step(cfg, g, k_new=g["k_new"], v_new=g["v_new"], qknorm=True)
    q2, kp, vp, _, _ = fused_append_ref(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                        d["slot_mapping"], d["context_lens"], d["gamma_q"],
                                        d["gamma_k"], cfg.eps, cfg.theta, block_size=BS)
    ref = attn_ref(q2, kp, vp, d["block_tables"], d["context_lens"], cfg.scale, block_size=BS)
    assert max_abs(out, ref) <= TOL_F16
    cfg, d = batch("c5", B=6, len_lo=1, len_hi=900, mbs=29, block_size=BS)
    g = to_device(d)
    out = _step(cfg, g)
    ref = attn_ref(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                   cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"], block_size=BS)
    assert max_abs(out, ref) <= TOL_E4M3


def test_step_block32_multi_token():
    cfg, d = batch("c2", B=7, len_lo=16, len_hi=700, mbs=22, block_size=BS)
    nq = 4
    rng = np.random.default_rng(3)
    q = rng.standard_normal((cfg.B, nq, cfg.Hq, cfg.D)).astype(np.float16)
    kn = rng.standard_normal((cfg.B, nq, cfg.Hkv, cfg.D)).astype(np.float16)
    vn = rng.standard_normal((cfg.B, nq, cfg.Hkv, cfg.D)).astype(np.float16)
    tab, lens = d["block_tables"], d["context_lens"]
    slots = np.array([int(tab[b, p // BS]) * BS + p % BS for b in range(cfg.B)
                      for p in range(int(lens[b]) - nq, int(lens[b]))], dtype=np.int64)
    g = to_device(d)
    out = _step(cfg, g, q=dev(q), k_new=dev(kn), v_new=dev(vn), nq=nq)
    kp, vp = append_ref(d["k_pool"], d["v_pool"], kn.reshape(-1, cfg.Hkv, cfg.D),
                        vn.reshape(-1, cfg.Hkv, cfg.D), slots, block_size=BS)
    assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
    ref = mq_attn_ref(q, kp, vp, tab, lens, cfg.scale, block_size=BS)
    assert max_abs(out, ref) <= TOL_F16


@pytest.mark.parametrize("fused", [False, True])
def test_append_block32(fused):
    cfg, d = batch("c4", B=9, len_lo=1, len_hi=500, mbs=16, block_size=BS)
    g = to_device(d)
    if fused:
        _lib.paged_kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["slot_mapping"],
                             q=g["q"], gamma_q=g["gamma_q"], gamma_k=g["gamma_k"],
                             context_lens=g["context_lens"], eps=cfg.eps, rope_theta=cfg.theta)
        _, kp, vp, _, _ = fused_append_ref(d["q"], d["k_new"], d["v_new"], d["k_pool"],
                                           d["v_pool"], d["slot_mapping"], d["context_lens"],
                                           d["gamma_q"], d["gamma_k"], cfg.eps, cfg.theta,
                                           block_size=BS)
        torch.cuda.synchronize()
        gk = g["k_pool"].cpu().numpy()
        assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))
        written = np.zeros(gk.shape[:3], dtype=bool)   # [NB, Hkv, BS]
        for slot in d["slot_mapping"]:
            written[slot // BS, :, slot % BS] = True
        assert np.array_equal(_u16(gk)[~written], _u16(kp)[~written])
        dk = np.abs(gk[written].astype(np.float64) - kp[written].astype(np.float64))
        ulp = np.spacing(np.maximum(np.abs(kp[written]), np.abs(gk[written])).astype(np.float16))
        assert np.all(dk <= ulp.astype(np.float64))
    else:
        _lib.paged_kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["slot_mapping"])
        kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], d["slot_mapping"],
                            block_size=BS)
        torch.cuda.synchronize()
        assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
        assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))


def test_copy_and_e4m3_append_block32():
    rng = np.random.default_rng(8)
    NB, Hkv, D = 300, 8, 128
    kp = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float16)
    vp = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float16)
    perm = rng.permutation(NB)
    src, dst = perm[:50].astype(np.int32), perm[50:100].astype(np.int32)
    gk, gv = dev(kp), dev(vp)
    _lib.paged_kv_copy_blocks(gk, gv, dev(src), dev(dst))
    torch.cuda.synchronize()
    rk, rv, _, _ = copy_blocks_ref(kp, vp, src, dst)
    assert np.array_equal(_u16(gk.cpu().numpy()), _u16(rk))
    assert np.array_equal(_u16(gv.cpu().numpy()), _u16(rv))
    # E4M3: rows 0..31 of 40 blocks, one call per row
    codes = np.zeros((NB, Hkv, BS, D), dtype=np.uint8)
    ks = np.zeros((NB, Hkv), dtype=np.float32)
    g = [dev(x) for x in (codes, codes.copy(), ks, ks.copy())]
    ref = (codes, codes.copy(), ks, ks.copy())
    blocks = perm[100:140]
    for r in range(BS):
        mag = rng.choice([0.01, 1.0, 50.0], size=(len(blocks), Hkv, 1))
        kn = (rng.standard_normal((len(blocks), Hkv, D)) * mag).astype(np.float16)
        vn = (rng.standard_normal((len(blocks), Hkv, D)) * mag).astype(np.float16)
        slots = (blocks * BS + r).astype(np.int64)
        _lib.paged_kv_append_e4m3(dev(kn), dev(vn), g[0], g[1], g[2], g[3], dev(slots))
        ref = append_e4m3_ref(*ref, kn, vn, slots, block_size=BS)
    torch.cuda.synchronize()
    for a, b in zip(g, ref):
        assert np.array_equal(np.ascontiguousarray(a.cpu().numpy()).view(np.uint8),
                              np.ascontiguousarray(b).view(np.uint8))


def test_decode_entry_points_reject_block32():
    cfg, d = batch("c2", B=3, len_lo=1, len_hi=200, mbs=7, block_size=BS)
    g = to_device(d)
    out = torch.empty_like(g["q"])
    with pytest.raises(_lib.PagedKVError):
        _lib.paged_attn_decode(out, g["q"], g["k_pool"], g["v_pool"], g["block_tables"],
                               g["context_lens"], cfg.scale)
