"""Seeded synthetic decode batches (inputs only; no attention arithmetic).

This module is the one place that both the HIP path's tests/bench and the CPU
oracle draw their inputs from.  It produces numpy arrays with the shapes and
value distributions of the five model-shaped decode layers below and holds
none of the method's arithmetic: no softmax, no normalisation, no rotation.

Structure of a batch (the pages' paging model: "Distributed LLM Inference
Serving Platform", section 2; "Roadmap: vLLM-style serving features for
TornadoVM batched decode", Serving / scheduling):
  * B sequences, each with L_b valid tokens (positions 0..L_b-1).
  * KV pools [NB, Hkv, 16, D]: physical blocks are handed out in the order
    of a seeded permutation of 0..NB-1, so a table row points at scattered
    blocks.  The last id of the permutation is a poison block; unused table
    entries point at it.
  * Every byte a correct kernel must not read holds NaN: rows past L_b in a
    sequence's last block, spare blocks and the poison block (fp16 0x7E00,
    E4M3 0x7F, scales NaN).
  * FP8 pools: the fp16 draw of each (block, kv head) tile is quantised to
    E4M3 with scale = amax(tile) / 448 (torch's float8_e4m3fn cast, which
    rounds to nearest even).  This is input preparation, done before the
    library ever sees the data.

Draw order per config (numpy default_rng(208000 + k) for config ck):
context_lens (and prefix tails) -> block permutation -> Q -> K -> V ->
(fused config) gamma_q, gamma_k, k_new, v_new.  Values are float32 N(0, 1)
rounded to fp16 (pool K/V: N(0, 1) times kv_sigma, 1 unless a test asks
for another data scale); gamma ~ N(1, 0.1) float32.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np

BLOCK_SIZE = 16
F16_NAN = np.array(0x7E00, dtype=np.uint16).view(np.float16)
E4M3_NAN = np.uint8(0x7F)
_CHUNK_BLOCKS = 2048


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    len_lo: int          # context length (after this step's append), inclusive
    len_hi: int
    mbs: int             # max blocks per sequence (table width)
    kv_dtype: str = "f16"            # "f16" or "e4m3"
    partition_size: int = 512        # 0 = single pass
    nb: int | None = None            # pool blocks; None = ceil(1.2 * need)
    prefix_tokens: int = 0           # shared prefix (multiple of 16)
    fused_append: bool = False       # Qwen3 QK-norm + RoPE before append
    theta: float = 1e6
    eps: float = 1e-6
    seed: int = 208000
    description: str = ""
    block_size: int = BLOCK_SIZE     # tokens per physical block (16 or 32)
    kv_sigma: float = 1.0            # K/V values are N(0, kv_sigma^2) before rounding

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_partitions(self) -> int:
        if self.partition_size == 0:
            return 1
        return -(-self.mbs * self.block_size // self.partition_size)

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c1": DecodeConfig(
        "c1", B=4, Hq=4, Hkv=2, D=64, len_lo=1, len_hi=64, mbs=4, nb=64,
        partition_size=0, seed=208001,
        description="tiny: B=4, 4 q / 2 kv heads, d=64, L~U[1,64], 64-block pool"),
    "c2": DecodeConfig(
        "c2", B=32, Hq=32, Hkv=8, D=128, len_lo=512, len_hi=4096, mbs=256,
        partition_size=512, seed=208002,
        description="LLaMA-3-8B-shaped layer: B=32, 32 q / 8 kv heads, d=128, "
                    "L~U[512,4096], fp16 KV"),
    "c3": DecodeConfig(
        "c3", B=128, Hq=32, Hkv=8, D=128, len_lo=16, len_hi=2048, mbs=192,
        prefix_tokens=1024, partition_size=512, seed=208003,
        description="Mistral-7B-shaped prefix-shared batch: B=128, 32/8 heads, "
                    "1024-token shared prefix + private tails U[16,2048]"),
    "c4": DecodeConfig(
        "c4", B=256, Hq=32, Hkv=8, D=128, len_lo=128, len_hi=8192, mbs=512,
        fused_append=True, partition_size=512, seed=208004,
        description="Qwen3-8B-shaped fused append+decode: B=256, 32/8 heads, "
                    "L~U[128,8192], RMSNorm eps 1e-6, RoPE theta 1e6"),
    "c5": DecodeConfig(
        "c5", B=64, Hq=64, Hkv=8, D=128, len_lo=3600, len_hi=4400, mbs=275,
        kv_dtype="e4m3", partition_size=512, seed=208005,
        description="70B-shaped long-context GQA, E4M3 KV with per-(block, kv "
                    "head) fp32 scales, 512-token partitions"),
}


def _normal_f16(rng, shape, sigma=1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return x.astype(np.float16)


def _quantise_e4m3(tiles_f16: np.ndarray):
    """fp16 tiles [n, Hkv, BS, D] -> (uint8 codes, float32 scales [n, Hkv])."""
    import torch  # torch's float8 cast is the input recipe's encoder

    x = torch.from_numpy(tiles_f16.astype(np.float32))
    amax = x.abs().amax(dim=(2, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (x / scale[:, :, None, None]).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale.numpy().astype(np.float32)


def generate(cfg: DecodeConfig, *, seed: int | None = None) -> dict:
    """Draw one decode batch for ``cfg``.  Returns a dict of numpy arrays.

    Keys: q [B,Hq,D] f16; k_pool, v_pool [NB,Hkv,16,D] (f16 or uint8);
    k_scale, v_scale [NB,Hkv] f32 (E4M3 only, else None); block_tables
    [B,MBS] int32; context_lens [B] int32; slot_mapping [B] int64 (slot of
    token L_b - 1); k_new, v_new [B,Hkv,D] f16 (the step's new rows);
    gamma_q, gamma_k [D] f32 (fused config only); poison_block int; nb int.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, Hkv, D, BS = cfg.B, cfg.Hkv, cfg.D, cfg.block_size

    lens = rng.integers(cfg.len_lo, cfg.len_hi, size=B, endpoint=True).astype(np.int64)
    if cfg.prefix_tokens:
        if cfg.prefix_tokens % BS:
            raise ValueError("prefix must be whole blocks")
        lens = lens + cfg.prefix_tokens
    prefix_blocks = cfg.prefix_tokens // BS
    own_blocks = -(-(lens - cfg.prefix_tokens) // BS)
    need = prefix_blocks + int(own_blocks.sum())
    nb = cfg.nb if cfg.nb is not None else math.ceil(1.2 * need)
    if need + 1 > nb:
        raise ValueError(f"pool of {nb} blocks cannot hold {need} + poison")
    if int(lens.max()) > cfg.mbs * BS:
        raise ValueError("context longer than the table allows")

    perm = rng.permutation(nb).astype(np.int64)
    poison = int(perm[-1])
    tables = np.full((B, cfg.mbs), poison, dtype=np.int32)
    cursor = 0
    prefix_ids = perm[cursor:cursor + prefix_blocks]
    cursor += prefix_blocks
    used = [prefix_ids]
    for b in range(B):
        n = int(own_blocks[b])
        ids = perm[cursor:cursor + n]
        cursor += n
        tables[b, :prefix_blocks] = prefix_ids
        tables[b, prefix_blocks:prefix_blocks + n] = ids
        used.append(ids)
    used_ids = np.concatenate(used)

    q = _normal_f16(rng, (B, cfg.Hq, D))

    fp8 = cfg.kv_dtype == "e4m3"
    pools, scales = [], []
    for _ in ("k", "v"):
        if fp8:
            pool = np.full((nb, Hkv, BS, D), E4M3_NAN, dtype=np.uint8)
            sc = np.full((nb, Hkv), np.nan, dtype=np.float32)
        else:
            pool = np.full((nb, Hkv, BS, D), F16_NAN, dtype=np.float16)
            sc = None
        for lo in range(0, len(used_ids), _CHUNK_BLOCKS):
            ids = used_ids[lo:lo + _CHUNK_BLOCKS]
            vals = _normal_f16(rng, (len(ids), Hkv, BS, D), cfg.kv_sigma)
            if fp8:
                codes, s = _quantise_e4m3(vals)
                pool[ids] = codes
                sc[ids] = s
            else:
                pool[ids] = vals
        pools.append(pool)
        scales.append(sc)

    # rows past the end of each sequence in its last block are poisoned
    nan = E4M3_NAN if fp8 else F16_NAN
    for b in range(B):
        L = int(lens[b])
        if L % BS:
            last = int(tables[b, (L - 1) // BS])
            for pool in pools:
                pool[last, :, L % BS:, :] = nan

    slot = np.array([int(tables[b, (int(lens[b]) - 1) // BS]) * BS + (int(lens[b]) - 1) % BS
                     for b in range(B)], dtype=np.int64)

    out = dict(q=q, k_pool=pools[0], v_pool=pools[1], k_scale=scales[0],
               v_scale=scales[1], block_tables=tables,
               context_lens=lens.astype(np.int32), slot_mapping=slot,
               poison_block=poison, nb=nb, gamma_q=None, gamma_k=None)
    if cfg.fused_append:
        out["gamma_q"] = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
        out["gamma_k"] = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    if not fp8:
        out["k_new"] = _normal_f16(rng, (B, Hkv, D))
        out["v_new"] = _normal_f16(rng, (B, Hkv, D))
        if cfg.fused_append:
            # the new token's slot holds poison until the append writes it
            for b in range(B):
                blk, off = divmod(int(slot[b]), BS)
                for pool in pools:
                    pool[blk, :, off, :] = F16_NAN
    else:
        out["k_new"] = out["v_new"] = None
    return out


def contiguous_layout(cfg: DecodeConfig, d: dict) -> dict:
    """The same batch with every sequence's blocks made physically
    consecutive: physical ids are handed out in order of first use in the
    tables (row by row), so a sequence's private blocks are adjacent and in
    logical order, and a shared prefix is stored once, ahead of the first
    sequence that uses it.  Unused table entries point at a poison block
    (the last id).  Same logical KV, same q and new rows: only the placement
    changes, which is what measures the cost of paging itself."""
    BS = cfg.block_size
    tables, lens = d["block_tables"], d["context_lens"]
    B = tables.shape[0]
    new_id = {}
    order = []
    for b in range(B):
        for i in range(-(-int(lens[b]) // BS)):
            old = int(tables[b, i])
            if old not in new_id:
                new_id[old] = len(order)
                order.append(old)
    used = len(order)
    poison = used
    out = dict(d)
    out["nb"] = used + 1
    out["poison_block"] = poison
    old_ids = np.asarray(order + [int(d["poison_block"])], dtype=np.int64)
    for key in ("k_pool", "v_pool", "k_scale", "v_scale"):
        if d.get(key) is not None:
            out[key] = np.ascontiguousarray(d[key][old_ids])
    t2 = np.full_like(tables, poison)
    for b in range(B):
        n = -(-int(lens[b]) // BS)
        t2[b, :n] = [new_id[int(x)] for x in tables[b, :n]]
    out["block_tables"] = t2
    out["slot_mapping"] = np.array(
        [int(t2[b, (int(lens[b]) - 1) // BS]) * BS + (int(lens[b]) - 1) % BS if lens[b] > 0
         else -1 for b in range(B)], dtype=np.int64)
    return out


def unique_kv_bytes(cfg: DecodeConfig, context_lens) -> int:
    """KV bytes of the distinct blocks a step reads: a shared prefix (every
    table maps the same prefix_tokens first) is counted once.  Equals
    kv_bytes when nothing is shared."""
    lens = np.asarray(context_lens, dtype=np.int64)
    if cfg.prefix_tokens <= 0 or lens.size == 0:
        return kv_bytes(cfg, lens)
    tails = np.maximum(lens - cfg.prefix_tokens, 0)
    return kv_bytes(cfg, np.concatenate([[cfg.prefix_tokens], tails]))


def kv_bytes(cfg: DecodeConfig, context_lens, window: int = 0) -> int:
    """Algorithmic KV bytes one decode step must read (K and V, plus scales).
    window > 0: only each sequence's last `window` tokens are read."""
    lens = np.asarray(context_lens, dtype=np.int64)
    if window > 0:
        lens = np.minimum(lens, window)
    tokens = int(np.sum(lens))
    elem = 1 if cfg.kv_dtype == "e4m3" else 2
    b = tokens * cfg.Hkv * cfg.D * 2 * elem
    if cfg.kv_dtype == "e4m3":
        tiles = int(np.sum(-(-lens // cfg.block_size)))
        b += tiles * cfg.Hkv * 2 * 4
    return b
