"""Several new query tokens per sequence in one step with more query columns
than one 16-wide product holds: a prefill chunk or a long speculative
verify ("Distributed LLM Inference Serving Platform", section 9.2: prefill
chunks of up to 512 tokens; "Roadmap: vLLM-style serving features for
TornadoVM batched decode", Deferred / WIP: chunked prefill, batch-prefill
verify).

The g * n_query columns of a (sequence, kv head) are split into 16-column
groups that each read the sequence's KV; new token j attends to positions
0 .. L - n_query + j.  The chunk's K/V rows are appended beforehand with
paged_kv_append (one slot per token), which also applies the Qwen3 QK-norm +
RoPE at each token's own position; the oracle is mq_attn_ref (and
fused_append_ref for the per-token prologue).
"""

import numpy as np
import pytest
import torch

from oracle import fused_append_ref, mq_attn_ref
from paged_kv_cache_208_amd import _lib

from helpers import TOL_E4M3, TOL_F16, batch, dev, max_abs, to_device

pytestmark = pytest.mark.gpu


def _chunk_step(cfg, g, q, nq, P=16):
    B, Hq, D = cfg.B, cfg.Hq, cfg.D
    out = torch.full((B, nq, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    ws = _lib.alloc_step_workspace(B, Hq * nq, cfg.Hkv, D, P)
    _lib.paged_decode_step(out, q, g["k_pool"], g["v_pool"], g["block_tables"],
                           g["context_lens"], cfg.scale, k_scale=g.get("k_scale"),
                           v_scale=g.get("v_scale"), partition_size=0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[3]).item() == 0, "arrival counters not reset"
    return out


@pytest.mark.parametrize("nq", [8, 64, 512])
def test_chunk_llama_shape(nq):
    cfg, d = batch("c2", B=2, len_lo=nq + 16, len_hi=nq + 700, mbs=(nq + 700) // 16 + 2,
                   seed=208_200 + nq)
    q = np.random.default_rng(nq).standard_normal((cfg.B, nq, cfg.Hq, cfg.D)).astype(np.float16)
    g = to_device(d)
    out = _chunk_step(cfg, g, dev(q), nq)
    ref = mq_attn_ref(q, d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                      cfg.scale)
    err = max_abs(out, ref)
    print(f"c2-shaped chunk nq={nq}: max_abs={err:.3e}", flush=True)
    assert err <= TOL_F16


@pytest.mark.parametrize("nq", [8, 64])
def test_chunk_70b_e4m3_shape(nq):
    cfg, d = batch("c5", B=2, len_lo=nq + 16, len_hi=nq + 600, mbs=(nq + 600) // 16 + 2,
                   seed=208_300 + nq)
    q = np.random.default_rng(nq + 1).standard_normal((cfg.B, nq, cfg.Hq, cfg.D)).astype(np.float16)
    g = to_device(d)
    out = _chunk_step(cfg, g, dev(q), nq)
    ref = mq_attn_ref(q, d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                      cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"])
    err = max_abs(out, ref)
    print(f"c5-shaped chunk nq={nq}: max_abs={err:.3e}", flush=True)
    assert err <= TOL_E4M3


def test_chunk_many_sequences_and_short_contexts():
    """B = 40 sequences (ranges cross many segment and column-group
    boundaries), contexts from exactly n_query tokens upwards."""
    nq = 16
    cfg, d = batch("c2", B=40, len_lo=nq, len_hi=nq + 300, mbs=(nq + 300) // 16 + 2,
                   seed=208_210)
    q = np.random.default_rng(3).standard_normal((cfg.B, nq, cfg.Hq, cfg.D)).astype(np.float16)
    g = to_device(d)
    out = _chunk_step(cfg, g, dev(q), nq, P=3)
    ref = mq_attn_ref(q, d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                      cfg.scale)
    assert max_abs(out, ref) <= TOL_F16


@pytest.mark.parametrize("nq", [8, 64])
def test_chunk_qwen3_qknorm_per_token_positions(nq):
    """Qwen3-shaped chunk: the fused append normalises and rotates every new
    token's q and k at its own position L - n_query + j and writes its k/v
    row; the step then attends with the causal mask."""
    cfg, d = batch("c4", B=3, len_lo=nq + 16, len_hi=nq + 500, mbs=(nq + 500) // 16 + 2,
                   seed=208_400 + nq)
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    rng = np.random.default_rng(nq + 2)
    q = rng.standard_normal((B, nq, Hq, D)).astype(np.float16)
    kn = rng.standard_normal((B, nq, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((B, nq, Hkv, D)).astype(np.float16)
    lens = d["context_lens"].astype(np.int64)
    tab = d["block_tables"]
    tok_lens = np.array([[L - nq + j + 1 for j in range(nq)] for L in lens], dtype=np.int32)
    slots = np.array([[int(tab[b, (p - 1) // 16]) * 16 + (p - 1) % 16 for p in tok_lens[b]]
                      for b in range(B)], dtype=np.int64)
    g = to_device(d)
    qd = dev(q.reshape(B * nq, Hq, D))
    _lib.paged_kv_append(dev(kn.reshape(B * nq, Hkv, D)), dev(vn.reshape(B * nq, Hkv, D)),
                         g["k_pool"], g["v_pool"], dev(slots.reshape(-1)), q=qd,
                         gamma_q=g["gamma_q"], gamma_k=g["gamma_k"],
                         context_lens=dev(tok_lens.reshape(-1)), eps=cfg.eps,
                         rope_theta=cfg.theta)
    out = _chunk_step(cfg, g, qd.view(B, nq, Hq, D), nq)
    q2, kp, vp, _, _ = fused_append_ref(q.reshape(B * nq, Hq, D), kn.reshape(B * nq, Hkv, D),
                                        vn.reshape(B * nq, Hkv, D), d["k_pool"], d["v_pool"],
                                        slots.reshape(-1), tok_lens.reshape(-1), d["gamma_q"],
                                        d["gamma_k"], cfg.eps, cfg.theta)
    ref = mq_attn_ref(q2.reshape(B, nq, Hq, D), kp, vp, tab, d["context_lens"], cfg.scale)
    err = max_abs(out, ref)
    print(f"c4-shaped chunk nq={nq} (per-token QK-norm): max_abs={err:.3e}", flush=True)
    assert err <= TOL_F16


@pytest.mark.parametrize("Hq,Hkv,nq", [(32, 8, 2), (16, 8, 4), (8, 8, 8)])
def test_step_qknorm_several_tokens_in_one_launch(Hq, Hkv, nq):
    """Up to 8 query columns: the one-launch step normalises and rotates
    every new token's q and k at its own position (L - n_query + j), appends
    the rows and attends causally."""
    cfg, d = batch("c4", B=5, Hq=Hq, Hkv=Hkv, len_lo=nq + 1, len_hi=700, mbs=46,
                   seed=208_500 + nq)
    B, D = cfg.B, cfg.D
    rng = np.random.default_rng(nq + 7)
    q = rng.standard_normal((B, nq, Hq, D)).astype(np.float16)
    kn = rng.standard_normal((B, nq, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((B, nq, Hkv, D)).astype(np.float16)
    lens = d["context_lens"].astype(np.int64)
    tab = d["block_tables"]
    tok_lens = np.array([[L - nq + j + 1 for j in range(nq)] for L in lens], dtype=np.int32)
    slots = np.array([[int(tab[b, (p - 1) // 16]) * 16 + (p - 1) % 16 for p in tok_lens[b]]
                      for b in range(B)], dtype=np.int64)
    g = to_device(d)
    qd = dev(q)
    out = torch.full((B, nq, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    ws = _lib.alloc_step_workspace(B, Hq * nq, Hkv, D, 16)
    _lib.paged_decode_step(out, qd, g["k_pool"], g["v_pool"], g["block_tables"],
                           g["context_lens"], cfg.scale, k_new=dev(kn), v_new=dev(vn),
                           gamma_q=g["gamma_q"], gamma_k=g["gamma_k"], eps=cfg.eps,
                           rope_theta=cfg.theta, partition_size=0, workspace=ws)
    torch.cuda.synchronize()
    q2, kp, vp, _, _ = fused_append_ref(q.reshape(B * nq, Hq, D), kn.reshape(B * nq, Hkv, D),
                                        vn.reshape(B * nq, Hkv, D), d["k_pool"], d["v_pool"],
                                        slots.reshape(-1), tok_lens.reshape(-1), d["gamma_q"],
                                        d["gamma_k"], cfg.eps, cfg.theta)
    # q' and the new k rows within one fp16 ulp of the once-rounded oracle,
    # v rows bitwise
    gq = qd.cpu().numpy().reshape(B * nq, Hq, D)
    ulp = np.spacing(np.maximum(np.abs(q2), np.abs(gq)).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(gq.astype(np.float64) - q2.astype(np.float64)) <= ulp)
    gk, gv = g["k_pool"].cpu().numpy(), g["v_pool"].cpu().numpy()
    assert np.array_equal(gv.view(np.uint16), vp.view(np.uint16))
    both_nan = np.isnan(gk) & np.isnan(kp)          # poisoned rows stay poisoned
    assert np.array_equal(np.isnan(gk), np.isnan(kp))
    dk = np.abs(gk[~both_nan].astype(np.float64) - kp[~both_nan].astype(np.float64))
    ulpk = np.spacing(np.maximum(np.abs(kp[~both_nan]), np.abs(gk[~both_nan]))
                      .astype(np.float16)).astype(np.float64)
    assert np.all(dk <= ulpk)
    ref = mq_attn_ref(q2.reshape(B, nq, Hq, D), kp, vp, tab, d["context_lens"], cfg.scale)
    err = max_abs(out, ref)
    print(f"QK-norm, {nq} tokens, g={Hq // Hkv}: max_abs={err:.3e}", flush=True)
    assert err <= TOL_F16
    assert torch.count_nonzero(ws[3]).item() == 0
