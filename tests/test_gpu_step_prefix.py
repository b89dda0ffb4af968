"""paged_decode_step with prefix_blocks > 0: every table starts with the same
physical blocks (a shared prompt prefix: "Roadmap: vLLM-style serving
features for TornadoVM batched decode", Serving / scheduling; "Distributed
LLM Inference Serving Platform", sections 2 and 11), and each prefix tile is
read once per group of 16 / g sequences.  Parity with the oracle (append
bitwise, attention within tolerance) across group sizes, head dims, E4M3,
32-token blocks, empty sequences and the smallest piece budget; the same
batch without the prefix argument agrees within rounding; repeated calls are
bitwise identical and leave the counters at zero."""

import numpy as np
import pytest
import torch

from oracle import append_ref, attn_ref
from paged_kv_cache_208_amd import _lib

from helpers import TOL_E4M3, TOL_F16, batch, dev, max_abs, sample_seqs, to_device

pytestmark = pytest.mark.gpu


def _u16(x):
    return np.ascontiguousarray(x).view(np.uint16)


def _run(cfg, g, *, prefix_blocks, append=True, P=16):
    B, Hq, D = g["q"].shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    ws = _lib.alloc_step_workspace(B, Hq, cfg.Hkv, D, P)
    kw = dict(k_new=g["k_new"], v_new=g["v_new"]) if append else {}
    _lib.paged_decode_step(out, g["q"], g["k_pool"], g["v_pool"], g["block_tables"],
                           g["context_lens"], cfg.scale, k_scale=g.get("k_scale"),
                           v_scale=g.get("v_scale"), partition_size=0,
                           prefix_blocks=prefix_blocks, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[3]).item() == 0, "arrival counters not reset"
    return out


def _check(cfg, d, out, g, append=True, seqs=None):
    kp, vp = d["k_pool"], d["v_pool"]
    if append:
        kp, vp = append_ref(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], cfg.block_size)
        assert np.array_equal(_u16(g["k_pool"].cpu().numpy()), _u16(kp))
        assert np.array_equal(_u16(g["v_pool"].cpu().numpy()), _u16(vp))
    ref = attn_ref(d["q"], kp, vp, d["block_tables"], d["context_lens"], cfg.scale,
                   k_scale=d.get("k_scale"), v_scale=d.get("v_scale"), block_size=cfg.block_size,
                   seqs=seqs)
    o = out.cpu().double().numpy()
    if seqs is not None:
        o, ref = o[seqs], ref[seqs]
    assert np.all(np.isfinite(o))
    return float(np.max(np.abs(o - ref)))


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 128), (16, 8, 128), (64, 8, 128),
                                      (16, 2, 64)])
def test_prefix_groups_parity(Hq, Hkv, D):
    """g = 4, 1, 2 and 8 (groups of 4, 16, 8 and 2 sequences), D = 64; B = 10
    leaves a partial last group."""
    cfg, d = batch("c3", B=10, Hq=Hq, Hkv=Hkv, D=D, prefix_tokens=64, len_lo=1, len_hi=300,
                   mbs=24, seed=208_600 + Hq + D)
    g = to_device(d)
    out = _run(cfg, g, prefix_blocks=4)
    err = _check(cfg, d, out, g)
    print(f"prefix g={Hq // Hkv} D={D}: max_abs={err:.3e}", flush=True)
    assert err <= TOL_F16


def test_prefix_full_size_mistral_shape():
    """The prefix-shared batch at full size (B = 128, 1024-token prefix),
    sampled sequences against the oracle."""
    cfg, d = batch("c3")
    g = to_device(d)
    out = _run(cfg, g, prefix_blocks=cfg.prefix_tokens // 16)
    seqs = sample_seqs(cfg.B, 8, seed=3)
    err = _check(cfg, d, out, g, seqs=seqs)
    print(f"c3 prefix step sampled {seqs}: max_abs={err:.3e}", flush=True)
    assert err <= TOL_F16


def test_prefix_agrees_with_the_plain_step_and_repeats_bitwise():
    cfg, d = batch("c3", B=13, prefix_tokens=128, len_lo=1, len_hi=400, mbs=34, seed=208_610)
    outs = []
    for _ in range(2):
        g = to_device(d)
        outs.append(_run(cfg, g, prefix_blocks=8))
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    g = to_device(d)
    plain = _run(cfg, g, prefix_blocks=0)
    assert float((outs[0].double() - plain.double()).abs().max()) <= 2 * TOL_F16


def test_prefix_e4m3():
    cfg, d = batch("c5", B=7, prefix_tokens=96, len_lo=1, len_hi=500, mbs=38, seed=208_620)
    g = to_device(d)
    out = _run(cfg, g, prefix_blocks=6, append=False)
    err = _check(cfg, d, out, g, append=False)
    print(f"prefix E4M3 (groups of 2): max_abs={err:.3e}", flush=True)
    assert err <= TOL_E4M3


def test_prefix_32_token_blocks():
    cfg, d = batch("c3", B=9, prefix_tokens=96, len_lo=1, len_hi=300, mbs=13, block_size=32,
                   seed=208_630)
    g = to_device(d)
    out = _run(cfg, g, prefix_blocks=3)
    err = _check(cfg, d, out, g)
    assert err <= TOL_F16


def test_prefix_empty_sequences_and_smallest_piece_budget():
    """Sequences with no tokens in the batch (zero rows, no pool writes),
    and max_partitions = 6 (three pieces per part) over many small ranges."""
    cfg, d = batch("c3", B=23, prefix_tokens=32, len_lo=1, len_hi=200, mbs=16, seed=208_640)
    lens = d["context_lens"].copy()
    empty = [0, 5, 6, 22]
    lens[empty] = 0
    slots = d["slot_mapping"].copy()
    slots[empty] = -1
    d2 = dict(d, context_lens=lens, slot_mapping=slots)
    g = to_device(d2)
    out = _run(cfg, g, prefix_blocks=2, P=6)
    err = _check(cfg, d2, out, g)
    assert err <= TOL_F16
    assert torch.all(out[empty] == 0)


def test_prefix_more_sequences_than_four_length_chunks():
    """B = 300: five chunks of 64 lengths in the scans that place each
    wave's range, with every seventh sequence empty."""
    cfg, d = batch("c3", B=300, prefix_tokens=32, len_lo=1, len_hi=100, mbs=9, seed=208_650)
    lens = d["context_lens"].copy()
    empty = list(range(0, 300, 7))
    lens[empty] = 0
    slots = d["slot_mapping"].copy()
    slots[empty] = -1
    d2 = dict(d, context_lens=lens, slot_mapping=slots)
    g = to_device(d2)
    out = _run(cfg, g, prefix_blocks=2, P=6)
    err = _check(cfg, d2, out, g)
    assert err <= TOL_F16
    assert torch.all(out[empty] == 0)
