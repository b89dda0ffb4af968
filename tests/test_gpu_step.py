"""GPU parity of paged_decode_step (append + decode + in-kernel combine in one
launch) against the fp64 oracle.

The step must equal paged_kv_append at each sequence's last slot followed by
paged_attn_decode and paged_attn_reduce: pools bitwise (plain append) or
within one fp16 ulp on the new k row (QK-norm), q' within one ulp, output
within the attention tolerance, and the arrival counters back at zero.
"""

import numpy as np
import pytest
import torch

from oracle import append_ref, attn_ref, fused_append_ref
from paged_kv_cache_208_amd import _lib

from helpers import TOL_E4M3, TOL_F16, batch, dev, max_abs, sample_seqs, to_device

pytestmark = pytest.mark.gpu


def _u16(x):
    return np.ascontiguousarray(x).view(np.uint16)


def _step(cfg, g, ps, *, append=True, qknorm=False, splits=16, window=0):
    """ps > 0: fixed partitions; ps == 0: balanced split into <= splits pieces."""
    B, Hq, D = g["q"].shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    P = _lib.max_partitions_for(cfg.mbs, ps) if ps else splits
    ws = _lib.alloc_step_workspace(B, Hq, cfg.Hkv, D, P)
    kw = {}
    if append:
        kw.update(k_new=g["k_new"], v_new=g["v_new"])
    if qknorm:
        kw.update(gamma_q=g["gamma_q"], gamma_k=g["gamma_k"], eps=cfg.eps, rope_theta=cfg.theta)
    _lib.paged_decode_step(out, g["q"], g["k_pool"], g["v_pool"], g["block_tables"],
                           g["context_lens"], cfg.scale, k_scale=g.get("k_scale"),
                           v_scale=g.get("v_scale"), partition_size=ps, window=window,
                           workspace=ws, **kw)
    torch.cuda.synchronize()
    return out, ws


@pytest.mark.parametrize("ps,splits", [(0, 3), (0, 16), (0, 64), (16, 0), (64, 0), (512, 0)])
def test_step_plain_append(ps, splits):
    cfg, d = batch("c2", B=6, len_lo=1, len_hi=700, mbs=44)
    g = to_device(d)
    out, ws = _step(cfg, g, ps, splits=splits)
    kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], d["slot_mapping"])
    assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
    assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))
    ref = attn_ref(d["q"], kp, vp, d["block_tables"], d["context_lens"], cfg.scale)
    assert max_abs(out, ref) <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0, "arrival counters not reset"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ps", [0, 64])
def test_step_qknorm(D, ps):
    kw = dict(B=7, len_lo=1, len_hi=1000, mbs=63)
    if D == 64:
        kw.update(D=64, Hq=16, Hkv=2)
    cfg, d = batch("c4", **kw)
    g = to_device(d)
    out, ws = _step(cfg, g, ps, qknorm=True)
    q2, kp, vp, _, _ = fused_append_ref(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                        d["slot_mapping"], d["context_lens"], d["gamma_q"],
                                        d["gamma_k"], cfg.eps, cfg.theta)
    gq = g["q"].cpu().numpy()
    ulp = np.spacing(np.maximum(np.abs(q2), np.abs(gq)).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(gq.astype(np.float64) - q2.astype(np.float64)) <= ulp)
    gk, gv = g["k_pool"].cpu().numpy(), g["v_pool"].cpu().numpy()
    assert np.array_equal(_u16(gv), _u16(vp))
    written = np.zeros(gk.shape[:3], dtype=bool)   # [NB, Hkv, BS]
    for slot in d["slot_mapping"]:
        written[slot // 16, :, slot % 16] = True
    assert np.array_equal(_u16(gk)[~written], _u16(kp)[~written])
    dk = np.abs(gk[written].astype(np.float64) - kp[written].astype(np.float64))
    ulpk = np.spacing(np.maximum(np.abs(kp[written]), np.abs(gk[written])).astype(np.float16))
    assert np.all(dk <= ulpk.astype(np.float64))
    ref = attn_ref(q2, kp, vp, d["block_tables"], d["context_lens"], cfg.scale)
    assert max_abs(out, ref) <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0


@pytest.mark.parametrize("ps", [0, 64, 512])
def test_step_e4m3_attend_and_combine(ps):
    cfg, d = batch("c5", B=4, len_lo=1, len_hi=900, mbs=57)
    g = to_device(d)
    out, _ = _step(cfg, g, ps, append=False)
    ref = attn_ref(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                   cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"])
    assert max_abs(out, ref) <= TOL_E4M3


def test_step_repeats_bitwise_and_matches_three_calls():
    """Counters left at zero let the next call combine again; the result is
    run-to-run identical and equals append + decode + reduce within
    rounding of the final division."""
    cfg, d = batch("c2", B=5, len_lo=1, len_hi=700, mbs=44)
    g = to_device(d)
    ws = _lib.alloc_step_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.D, 16)
    outs = []
    for ps in (0, 0, 0):
        out = torch.empty_like(g["q"])
        _lib.paged_decode_step(out, g["q"], g["k_pool"], g["v_pool"], g["block_tables"],
                               g["context_lens"], cfg.scale, k_new=g["k_new"], v_new=g["v_new"],
                               partition_size=ps, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    g2 = to_device(d)
    _lib.paged_kv_append(g2["k_new"], g2["v_new"], g2["k_pool"], g2["v_pool"], g2["slot_mapping"])
    ref = torch.empty_like(g2["q"])
    _lib.decode_step(ref, g2["q"], g2["k_pool"], g2["v_pool"], g2["block_tables"],
                     g2["context_lens"], cfg.scale, partition_size=64)
    torch.cuda.synchronize()
    diff = (outs[0].double() - ref.double()).abs().max().item()
    assert diff <= 2e-3


@pytest.mark.parametrize("ps", [0, 64])
def test_step_empty_and_single_token_contexts(ps):
    cfg, d = batch("c2", B=5, len_lo=1, len_hi=300, mbs=19)
    lens = d["context_lens"].copy()
    lens[0] = 0
    lens[3] = 1
    tab = d["block_tables"]
    slots = d["slot_mapping"].copy()
    slots[0] = -1
    slots[3] = int(tab[3, 0]) * 16
    d2 = dict(d, context_lens=lens, slot_mapping=slots)
    g = to_device(d2)
    out, ws = _step(cfg, g, ps)
    kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], slots)
    assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
    assert torch.all(out[0] == 0)
    # one token: the output is that token's (new) value row
    v3 = torch.from_numpy(d["v_new"][3]).cuda().repeat_interleave(cfg.group, dim=0)
    assert torch.equal(out[3].view(torch.int16), v3.view(torch.int16))
    ref = attn_ref(d["q"], kp, vp, tab, lens, cfg.scale)
    assert max_abs(out, ref) <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("balanced", [True, False])
def test_step_full_size_sampled(name, balanced):
    cfg, d = batch(name)
    g = to_device(d)
    fp8 = cfg.kv_dtype == "e4m3"
    out, ws = _step(cfg, g, 0 if balanced else cfg.partition_size, append=not fp8,
                    qknorm=cfg.fused_append)
    o = out.cpu().double().numpy()
    assert np.all(np.isfinite(o))
    seqs = sample_seqs(cfg.B, 5, seed=3)
    if fp8:
        ref = attn_ref(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                       cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"], seqs=seqs)[seqs]
        tol = TOL_E4M3
    elif cfg.fused_append:
        q2, kp, vp, _, _ = fused_append_ref(d["q"][seqs], d["k_new"][seqs], d["v_new"][seqs],
                                            d["k_pool"], d["v_pool"], d["slot_mapping"][seqs],
                                            d["context_lens"][seqs], d["gamma_q"], d["gamma_k"],
                                            cfg.eps, cfg.theta)
        ref = attn_ref(q2, kp, vp, d["block_tables"][seqs], d["context_lens"][seqs], cfg.scale)
        tol = TOL_F16
    else:
        kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"][seqs], d["v_new"][seqs],
                            d["slot_mapping"][seqs])
        ref = attn_ref(d["q"][seqs], kp, vp, d["block_tables"][seqs], d["context_lens"][seqs],
                       cfg.scale)
        tol = TOL_F16
    err = float(np.max(np.abs(o[seqs] - ref)))
    print(f"{name} step sampled {seqs} max_abs={err:.3e}", flush=True)
    assert err <= tol
    assert torch.count_nonzero(ws[3]).item() == 0


def _relen(d, lens):
    """The batch with new context lengths: the new token moves to each
    sequence's new last position (no slot for an empty sequence)."""
    lens = np.asarray(lens, dtype=np.int32)
    tab = d["block_tables"]
    slots = np.array([int(tab[b, (n - 1) // 16]) * 16 + (n - 1) % 16 if n > 0 else -1
                      for b, n in enumerate(lens)], dtype=np.int64)
    return dict(d, context_lens=lens, slot_mapping=slots)


@pytest.mark.parametrize("B", [100, 300])
@pytest.mark.parametrize("splits", [3, 16])
def test_step_balanced_many_short_sequences(splits, B):
    """More sequences than one wave scans at once (B > 64, up to five
    chunks of 64 lengths), segments of 1-3 tiles so one wave's range holds
    many segments, every fifth sequence empty."""
    cfg, d = batch("c2", B=B, len_lo=1, len_hi=48, mbs=3)
    lens = d["context_lens"].copy()
    lens[::5] = 0
    d2 = _relen(d, lens)
    g = to_device(d2)
    out, ws = _step(cfg, g, 0, splits=splits)
    kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], d2["slot_mapping"])
    assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
    assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))
    ref = attn_ref(d["q"], kp, vp, d["block_tables"], lens, cfg.scale)
    assert torch.all(out[::5] == 0)
    assert max_abs(out, ref) <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 128), (16, 8, 64), (64, 8, 128), (8, 4, 64)])
def test_step_balanced_group_sizes(Hq, Hkv, D):
    cfg, d = batch("c2", B=9, Hq=Hq, Hkv=Hkv, D=D, len_lo=1, len_hi=900, mbs=57)
    g = to_device(d)
    out, ws = _step(cfg, g, 0)
    kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], d["slot_mapping"])
    assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
    ref = attn_ref(d["q"], kp, vp, d["block_tables"], d["context_lens"], cfg.scale)
    assert max_abs(out, ref) <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0


@pytest.mark.parametrize("D", [64, 128])
def test_step_balanced_e4m3_with_empty_sequences(D):
    kw = dict(B=70, len_lo=1, len_hi=300, mbs=19)
    if D == 64:
        kw.update(D=64, Hq=16, Hkv=2)
    cfg, d = batch("c5", **kw)
    lens = d["context_lens"].copy()
    lens[3::9] = 0
    d2 = dict(d, context_lens=lens)
    g = to_device(d2)
    out, ws = _step(cfg, g, 0, append=False)
    ref = attn_ref(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], lens, cfg.scale,
                   k_scale=d["k_scale"], v_scale=d["v_scale"])
    assert torch.all(out[3::9] == 0)
    assert max_abs(out, ref) <= TOL_E4M3
    assert torch.count_nonzero(ws[3]).item() == 0


def test_step_balanced_qknorm_many_sequences():
    """QK-norm + RoPE with B > 64, empty sequences and short segments: angle
    tables change between neighbouring segments of one wave."""
    cfg, d = batch("c4", B=80, len_lo=1, len_hi=200, mbs=13)
    lens = d["context_lens"].copy()
    lens[::7] = 0
    d2 = _relen(d, lens)
    g = to_device(d2)
    out, ws = _step(cfg, g, 0, qknorm=True)
    q2, kp, vp, _, _ = fused_append_ref(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                        d2["slot_mapping"], lens, d["gamma_q"], d["gamma_k"],
                                        cfg.eps, cfg.theta)
    gq = g["q"].cpu().numpy()
    live = lens > 0
    ulp = np.spacing(np.maximum(np.abs(q2), np.abs(gq)).astype(np.float16)).astype(np.float64)
    assert np.all((np.abs(gq.astype(np.float64) - q2.astype(np.float64)) <= ulp)[live])
    assert np.array_equal(_u16(gq[~live]), _u16(d["q"][~live])), "q of empty sequences changed"
    assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))
    ref = attn_ref(q2, kp, vp, d["block_tables"], lens, cfg.scale)
    assert torch.all(out[::7] == 0)
    assert max_abs(out, ref) <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0


@pytest.mark.parametrize("window", [1, 15, 16, 17, 100, 1000])
def test_step_sliding_window(window):
    """Only the last `window` tokens are attended; blocks before the window
    hold NaN here, so reading any of them would show."""
    cfg, d = batch("c2", B=9, len_lo=1, len_hi=700, mbs=44)
    lens = d["context_lens"]
    kp0, vp0 = d["k_pool"].copy(), d["v_pool"].copy()
    tab = d["block_tables"]
    for b, L in enumerate(lens):                     # poison whole blocks before the window
        start = max(0, int(L) - window) // 16 if window < L else 0
        for n in range(start):
            kp0[tab[b, n]] = np.float16(np.nan)
            vp0[tab[b, n]] = np.float16(np.nan)
    d2 = dict(d, k_pool=kp0, v_pool=vp0)
    g = to_device(d2)
    out, ws = _step(cfg, g, 0, window=window)
    kp, vp = append_ref(kp0, vp0, d["k_new"], d["v_new"], d["slot_mapping"])
    ref = attn_ref(d["q"], kp, vp, tab, lens, cfg.scale, window=window)
    assert max_abs(out, ref) <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0


def test_step_sliding_window_qknorm_and_e4m3():
    cfg, d = batch("c4", B=7, len_lo=1, len_hi=1000, mbs=63)
    g = to_device(d)
    out, _ = _step(cfg, g, 0, qknorm=True, window=300)
    q2, kp, vp, _, _ = fused_append_ref(d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                        d["slot_mapping"], d["context_lens"], d["gamma_q"],
                                        d["gamma_k"], cfg.eps, cfg.theta)
    ref = attn_ref(q2, kp, vp, d["block_tables"], d["context_lens"], cfg.scale, window=300)
    assert max_abs(out, ref) <= TOL_F16
    cfg, d = batch("c5", B=6, len_lo=1, len_hi=900, mbs=57)
    g = to_device(d)
    out, _ = _step(cfg, g, 0, append=False, window=129)
    ref = attn_ref(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                   cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"], window=129)
    assert max_abs(out, ref) <= TOL_E4M3


def _multi_token(cfg, d, nq, seed):
    """nq new tokens per sequence at positions L - nq .. L - 1."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    q = rng.standard_normal((B, nq, Hq, D)).astype(np.float16)
    kn = rng.standard_normal((B, nq, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((B, nq, Hkv, D)).astype(np.float16)
    tab, lens = d["block_tables"], d["context_lens"]
    slots = np.array([int(tab[b, p // 16]) * 16 + p % 16
                      for b in range(B) for p in range(int(lens[b]) - nq, int(lens[b]))],
                     dtype=np.int64)
    return q, kn, vn, slots


@pytest.mark.parametrize("nq,Hq,Hkv,D", [(2, 32, 8, 128), (4, 32, 8, 128), (16, 8, 8, 64),
                                         (2, 64, 8, 128), (8, 16, 8, 64)])
def test_step_multi_token_causal(nq, Hq, Hkv, D):
    """Several new tokens per sequence share every KV byte read: appended
    rows (which may straddle two tiles of different waves' ranges) are
    bitwise those of the separate append, and token j attends causally."""
    from oracle import mq_attn_ref
    cfg, d = batch("c2", B=7, Hq=Hq, Hkv=Hkv, D=D, len_lo=16, len_hi=700, mbs=44)
    q, kn, vn, slots = _multi_token(cfg, d, nq, seed=70 + nq)
    g = to_device(d)
    B = cfg.B
    out = torch.full((B, nq, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    ws = _lib.alloc_step_workspace(B, Hq * nq, Hkv, D, 16)
    _lib.paged_decode_step(out, dev(q), g["k_pool"], g["v_pool"], g["block_tables"],
                           g["context_lens"], cfg.scale, k_new=dev(kn), v_new=dev(vn),
                           partition_size=0, workspace=ws)
    torch.cuda.synchronize()
    kp, vp = append_ref(d["k_pool"], d["v_pool"], kn.reshape(B * nq, Hkv, D),
                        vn.reshape(B * nq, Hkv, D), slots)
    assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
    assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))
    ref = mq_attn_ref(q, kp, vp, d["block_tables"], d["context_lens"], cfg.scale)
    assert max_abs(out, ref) <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0


def test_step_multi_token_e4m3():
    from oracle import mq_attn_ref
    cfg, d = batch("c5", B=5, len_lo=16, len_hi=900, mbs=57)
    nq = 2
    q, _, _, _ = _multi_token(cfg, d, nq, seed=5)
    g = to_device(d)
    out = torch.empty((cfg.B, nq, cfg.Hq, cfg.D), dtype=torch.float16, device="cuda")
    ws = _lib.alloc_step_workspace(cfg.B, cfg.Hq * nq, cfg.Hkv, cfg.D, 16)
    _lib.paged_decode_step(out, dev(q), g["k_pool"], g["v_pool"], g["block_tables"],
                           g["context_lens"], cfg.scale, k_scale=g["k_scale"],
                           v_scale=g["v_scale"], partition_size=0, workspace=ws)
    torch.cuda.synchronize()
    ref = mq_attn_ref(q, d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                      cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"])
    assert max_abs(out, ref) <= TOL_E4M3


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (16, 2), (32, 8)])
def test_step_balanced_head_wrap_with_empty_ends(Hq, Hkv):
    """The balanced split orders tiles kv head first: a wave's range runs from
    the last sequences of one head into the first sequences of the next.
    Empty sequences at both ends of the batch (and B > 64) make the cursor
    skip them across that wrap; splits=3 makes the ranges long enough to
    cross several heads."""
    cfg, d = batch("c2", B=70, Hq=Hq, Hkv=Hkv, D=128, len_lo=1, len_hi=120, mbs=8)
    lens = d["context_lens"].copy()
    lens[[0, 1, 35, 68, 69]] = 0
    keep = lens > 0
    slots = np.where(keep, d["slot_mapping"], -1)
    d2 = dict(d, context_lens=lens)
    for splits in (3, 16):
        g = to_device(d2)
        out, ws = _step(cfg, g, 0, splits=splits)
        kp, vp = append_ref(d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], slots)
        assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
        assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))
        ref = attn_ref(d["q"], kp, vp, d["block_tables"], lens, cfg.scale)
        assert torch.all(out[~torch.from_numpy(keep).cuda()] == 0)
        assert max_abs(out, ref) <= TOL_F16
        assert torch.count_nonzero(ws[3]).item() == 0
