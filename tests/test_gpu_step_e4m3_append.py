"""paged_decode_step over E4M3 pools with k_new: each sequence's new row goes
to position L - 1 through the E4M3 append policy ("Roadmap: vLLM-style
serving features for TornadoVM batched decode", Sampling / logits: a
quantized KV cache; the policy keeps each block's scale at the running amax
of its rows / 448 and re-encodes earlier rows when it grows), then the step
attends.  Pools and scales must equal the oracle's append (append_e4m3_ref,
with the slots the tables give) bit for bit, the output must match attn_ref
on the appended pools within the E4M3 tolerance, and the same step done as
paged_kv_append_e4m3 followed by the step without k_new gives the same bits."""

import numpy as np
import pytest
import torch

from oracle import append_e4m3_ref, attn_ref
from paged_kv_cache_208_amd import _lib

from helpers import TOL_E4M3, batch, dev, max_abs, to_device

pytestmark = pytest.mark.gpu


def _slots(d, BS):
    tab, lens = d["block_tables"], d["context_lens"].astype(np.int64)
    return np.array([int(tab[b, (L - 1) // BS]) * BS + (L - 1) % BS if L > 0 else -1
                     for b, L in enumerate(lens)], dtype=np.int64)


def _step(cfg, g, kn, vn, P=16):
    B, Hq, D = g["q"].shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    ws = _lib.alloc_step_workspace(B, Hq, cfg.Hkv, D, P)
    _lib.paged_decode_step(out, g["q"], g["k_pool"], g["v_pool"], g["block_tables"],
                           g["context_lens"], cfg.scale, k_scale=g["k_scale"],
                           v_scale=g["v_scale"], k_new=kn, v_new=vn, partition_size=0,
                           workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[3]).item() == 0
    return out


@pytest.mark.parametrize("B,len_lo,len_hi,bs,seed", [(16, 100, 600, 16, 1), (9, 1, 70, 16, 2),
                                                     (7, 33, 300, 32, 3)])
def test_step_appends_e4m3_rows_like_the_oracle(B, len_lo, len_hi, bs, seed):
    cfg, d = batch("c5", B=B, len_lo=len_lo, len_hi=len_hi, mbs=len_hi // bs + 2, block_size=bs,
                   seed=208_700 + seed)
    rng = np.random.default_rng(seed)
    kn = (3.0 * rng.standard_normal((B, cfg.Hkv, cfg.D))).astype(np.float16)  # often raises the scale
    vn = rng.standard_normal((B, cfg.Hkv, cfg.D)).astype(np.float16)
    g = to_device(d)
    out = _step(cfg, g, dev(kn), dev(vn))
    ref = append_e4m3_ref(d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"], kn, vn,
                          _slots(d, bs), block_size=bs)
    got = [g[k].cpu().numpy() for k in ("k_pool", "v_pool", "k_scale", "v_scale")]
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    assert np.array_equal(got[2].view(np.uint32), ref[2].view(np.uint32))
    assert np.array_equal(got[3].view(np.uint32), ref[3].view(np.uint32))
    ref_out = attn_ref(d["q"], ref[0], ref[1], d["block_tables"], d["context_lens"], cfg.scale,
                       k_scale=ref[2], v_scale=ref[3], block_size=bs)
    err = max_abs(out, ref_out)
    print(f"E4M3 step with append B={B} BS={bs}: max_abs={err:.3e}", flush=True)
    assert err <= TOL_E4M3


def test_step_append_equals_the_two_calls():
    cfg, d = batch("c5", B=12, len_lo=1, len_hi=400, mbs=27, seed=208_710)
    rng = np.random.default_rng(7)
    kn = rng.standard_normal((cfg.B, cfg.Hkv, cfg.D)).astype(np.float16)
    vn = rng.standard_normal((cfg.B, cfg.Hkv, cfg.D)).astype(np.float16)
    g1 = to_device(d)
    out1 = _step(cfg, g1, dev(kn), dev(vn))
    g2 = to_device(d)
    _lib.paged_kv_append_e4m3(dev(kn), dev(vn), g2["k_pool"], g2["v_pool"], g2["k_scale"],
                              g2["v_scale"], dev(_slots(d, 16)))
    out2 = _step(cfg, g2, None, None)
    for k in ("k_pool", "v_pool", "k_scale", "v_scale"):
        assert torch.equal(g1[k].view(torch.uint8), g2[k].view(torch.uint8)), k
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
