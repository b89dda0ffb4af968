"""Seeded input generator: structure of the synthetic decode batches."""

import numpy as np
import pytest

from paged_kv_cache_208_amd import synth


def _small(name, **kw):
    cfg = synth.CONFIGS[name]
    shrink = dict(c2=dict(B=4), c3=dict(B=4), c4=dict(B=4, len_hi=700), c5=dict(B=3))
    return cfg.replace(**{**shrink.get(name, {}), **kw})


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_structure(name):
    cfg = _small(name)
    d = synth.generate(cfg)
    B, BS = cfg.B, 16
    lens, tab = d["context_lens"], d["block_tables"]
    assert lens.dtype == np.int32 and tab.dtype == np.int32
    assert np.all(lens >= cfg.len_lo + cfg.prefix_tokens)
    assert np.all(lens <= cfg.len_hi + cfg.prefix_tokens)
    used = []
    for b in range(B):
        n = -(-int(lens[b]) // BS)
        assert np.all(tab[b, n:] == d["poison_block"])
        used.extend(tab[b, cfg.prefix_tokens // BS:n].tolist())
    assert len(set(used)) == len(used), "private blocks are never shared"
    assert d["poison_block"] not in used
    # slot of the newest token = block * 16 + row
    for b in range(B):
        t = int(lens[b]) - 1
        assert d["slot_mapping"][b] == tab[b, t // BS] * BS + t % BS
    pool = d["k_pool"]
    if cfg.kv_dtype == "e4m3":
        assert pool.dtype == np.uint8
        assert np.all(pool[d["poison_block"]] == 0x7F)
        assert np.isnan(d["k_scale"][d["poison_block"]]).all()
        assert np.all(d["k_scale"][used] > 0)
    else:
        assert np.isnan(pool[d["poison_block"]].astype(np.float32)).all()
    # pad rows past L in the last block are poisoned, valid rows are finite
    for b in range(B):
        L = int(lens[b])
        last = tab[b, (L - 1) // BS]
        rows = pool[last, :, :L % BS or BS].astype(np.float32)
        if cfg.kv_dtype == "e4m3":
            assert np.all(pool[last, :, L % BS:] == 0x7F) if L % BS else True
        else:
            if cfg.fused_append:
                rows = rows[:, :-1]    # newest slot is poisoned until appended
            assert np.all(np.isfinite(rows))
            if L % BS:
                assert np.isnan(pool[last, :, L % BS:].astype(np.float32)).all()


def test_prefix_is_shared_by_every_table():
    cfg = _small("c3")
    d = synth.generate(cfg)
    nb = cfg.prefix_tokens // 16
    assert np.all(d["block_tables"][:, :nb] == d["block_tables"][0, :nb])


def test_seeded_and_reproducible():
    cfg = _small("c2")
    a, b = synth.generate(cfg), synth.generate(cfg)
    for k in ("q", "k_pool", "block_tables", "context_lens"):
        np.testing.assert_array_equal(a[k].view(np.uint8), b[k].view(np.uint8))
    c = synth.generate(cfg, seed=1)
    assert not np.array_equal(a["context_lens"], c["context_lens"])


def test_e4m3_scales_cover_the_tile():
    cfg = _small("c5")
    d = synth.generate(cfg)
    import torch
    b0 = d["block_tables"][0, 0]
    vals = torch.from_numpy(d["k_pool"][b0]).view(torch.float8_e4m3fn).float().numpy()
    assert np.nanmax(np.abs(vals)) == 448.0       # the amax element maps to 448


def test_kv_bytes():
    cfg = synth.CONFIGS["c2"]
    assert synth.kv_bytes(cfg, [10, 6]) == 16 * 8 * 128 * 2 * 2
    assert synth.kv_bytes(synth.CONFIGS["c5"], [16]) == 16 * 8 * 128 * 2 + 8 * 2 * 4


def test_contiguous_layout_keeps_the_logical_kv_and_packs_each_sequence():
    """The relayout used to price paging: every sequence reads the same
    logical rows, its private blocks are consecutive and ascending, a shared
    prefix is stored once, and the new slots point at the same logical
    position (L - 1)."""
    cfg = synth.CONFIGS["c3"].replace(B=6, len_hi=100, mbs=70)
    d = synth.generate(cfg)
    c = synth.contiguous_layout(cfg, d)
    prefix = cfg.prefix_tokens // 16
    for b in range(cfg.B):
        L = int(d["context_lens"][b])
        n = -(-L // 16)
        old = d["k_pool"][d["block_tables"][b, :n]].view(np.uint16)
        new = c["k_pool"][c["block_tables"][b, :n]].view(np.uint16)
        assert np.array_equal(old, new)
        own = c["block_tables"][b, prefix:n]
        assert np.all(np.diff(own) == 1)
        assert np.all(c["block_tables"][b, n:] == c["poison_block"])
        s = int(c["slot_mapping"][b])
        assert c["block_tables"][b, (L - 1) // 16] == s // 16 and s % 16 == (L - 1) % 16
    assert np.array_equal(c["block_tables"][:, :prefix], np.tile(np.arange(prefix), (cfg.B, 1)))
    assert c["nb"] == prefix + sum(-(-(int(L) - cfg.prefix_tokens) // 16)
                                   for L in d["context_lens"]) + 1


def test_unique_kv_bytes_counts_a_shared_prefix_once():
    cfg = synth.CONFIGS["c3"]
    lens = np.array([1024 + 16, 1024 + 100, 1024 + 2048])
    per_token = cfg.Hkv * cfg.D * 2 * 2
    assert synth.kv_bytes(cfg, lens) == int(lens.sum()) * per_token
    assert synth.unique_kv_bytes(cfg, lens) == (1024 + 16 + 100 + 2048) * per_token
    c2 = synth.CONFIGS["c2"]
    assert synth.unique_kv_bytes(c2, lens) == synth.kv_bytes(c2, lens)   # nothing shared
