#!/usr/bin/env python3
"""Batched-decode PagedAttention benchmark on one MI355X.

One step = one decode step of one attention layer over a synthetic batch:
  * fp16 configs: this step's K/V row of every sequence is written to its
    slot, then each query attends over its paged KV in split-context
    partitions, which are combined into the output
  * fused config (c4): the append also applies QK-RMSNorm + RoPE to q and k
  * E4M3 config (c5): attention over FP8 KV + combine
By default the step is one launch of paged_decode_step; --unfused times the
same work as paged_kv_append -> paged_attn_decode -> paged_attn_reduce on
one HIP stream.  Inputs are resident in HBM before timing starts;
R rotated copies of the pools, tables and q (>= 1 GiB touched between
reuses) keep the 256 MB last-level cache from serving the KV.

Prints one JSON line: value = KV-read GB/s over the whole step
(algorithmic KV bytes / step time), plus steps/s, tokens/s, the decode
kernel's roofline position (its own HIP-event time) and the CPU oracle
baseline timed on this host.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from paged_kv_cache_208_amd import synth  # noqa: E402
from paged_kv_cache_208_amd.roofline import HBM_GBPS  # noqa: E402

METRIC = "paged decode attention KV-read GB/s (% of HBM peak) + decode steps/s at B"
ROTATE_BYTES = 1 << 30

# HBM bytes per step of the balanced step (its attend launch plus, without
# QK-norm, its combine launch), from two rocprofv3 passes (FETCH_SIZE,
# WRITE_SIZE in KiB per dispatch), each scaled by what the counter reads for a
# plain 256 MiB copy (x2.0 and x1.0).  Keyed by workload and a hash of the step
# kernels' code (their sources without comments): a changed kernel reports
# traffic null until it is measured again.
STEP_SOURCES = ("decode_stream.hip", "decode_stream_cached.hip", "decode_stream_impl.h",
                "decode_tile.h", "device.h", "kernels.h", "shape_limits.h")
# the shared-prefix step's own sources (its key hashes both sets)
PREFIX_SOURCES = ("decode_stream_prefix.hip", "decode_prefix_impl.h")
# The key's last two fields are the shared-blocks hint and the shared prefix
# (in blocks) that the run passed; its hash covers the plain step's sources,
# and the prefix step's too for a shared-prefix run.
MEASURED_TRAFFIC = {
    ("c2", "a3378f8d27623030", False, 0): {"fetch_bytes": 316610251, "write_bytes": 3080192,
        "attend_fetch_bytes": 313798347, "combine_fetch_bytes": 2811904,
        "source": "profiles/step_hbm_bytes.md"},
    ("c3", "aca093285485677a", False, 64): {"fetch_bytes": 592490944, "write_bytes": 9240576,
        "attend_fetch_bytes": 584521152, "combine_fetch_bytes": 7969792,
        "source": "profiles/step_hbm_bytes.md"},
    ("c3", "a3378f8d27623030", True, 0): {"fetch_bytes": 570523627, "write_bytes": 5795203,
        "attend_fetch_bytes": 566065131, "combine_fetch_bytes": 4458496,
        "source": "profiles/step_hbm_bytes.md"},
    ("c4", "a3378f8d27623030", False, 0): {"fetch_bytes": 4285652896, "write_bytes": 10022176,
        "attend_fetch_bytes": 4285652896, "combine_fetch_bytes": 0,
        "source": "profiles/step_hbm_bytes.md"},
    ("c5", "a3378f8d27623030", False, 0): {"fetch_bytes": 563634560, "write_bytes": 11803403,
        "attend_fetch_bytes": 552571264, "combine_fetch_bytes": 11063296,
        "source": "profiles/step_hbm_bytes.md"},
}




def code_of(text):
    """A source's code without its // comments and blank lines (so that a
    comment-only edit keeps the measured traffic)."""
    lines = []
    for ln in text.splitlines():
        ln = ln.split("//", 1)[0].rstrip()
        if ln.strip():
            lines.append(ln)
    return "\n".join(lines)


def step_source_hash(read=None, prefix=False):
    import hashlib
    h = hashlib.sha256()
    for name in STEP_SOURCES + (PREFIX_SOURCES if prefix else ()):
        path = os.path.join("paged_kv_cache_208_amd", "csrc", name)
        if read is None:
            with open(os.path.join(ROOT, path)) as f:
                text = f.read()
        else:
            text = read(path)
        h.update(code_of(text).encode())
    return h.hexdigest()[:16]


def step_tile_ids(cfg, d, nq, prefix_blocks, cached):
    """The (block, kv head) tiles the balanced step reads, in its order (kv
    head, then sequence, then column group, then tile; with a shared prefix,
    per kv head the prefix once per group of 16 / g sequences, then each
    sequence's own tiles), as int32 tile indices for pkv_tile_read (~index:
    read with the default cache policy, as the step does for every tile
    under the shared-blocks hint)."""
    tab, lens = d["block_tables"], d["context_lens"].astype(np.int64)
    g = cfg.Hq // cfg.Hkv
    hb = cfg.block_size // 16                      # tiles per block
    cg = 1 if g * nq <= 16 else -(-g * nq // 16)   # 16-column groups per sequence
    ntile = -(-lens // 16)

    def seq_tiles(b, kvh, lo, hi):
        n = np.arange(lo, hi)
        return (tab[b, n // hb].astype(np.int64) * cfg.Hkv + kvh) * hb + n % hb

    out = []
    for kvh in range(cfg.Hkv):
        if prefix_blocks:
            tp = prefix_blocks * hb
            spp = 16 // g
            for lead in range(0, cfg.B, spp):
                t = seq_tiles(lead, kvh, 0, tp)
                out.append(~t if cached else t)
            for b in range(cfg.B):
                if ntile[b] > tp:
                    t = seq_tiles(b, kvh, tp, ntile[b])
                    out.append(~t if cached else t)
        else:
            for b in range(cfg.B):
                t = seq_tiles(b, kvh, 0, ntile[b])
                for _ in range(cg):
                    out.append(~t if cached else t)
    return np.concatenate(out).astype(np.int32)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="c2", choices=sorted(synth.CONFIGS))
    p.add_argument("--partition-size", type=int, default=None)
    p.add_argument("--rotate", type=int, default=None, help="copies of the inputs (default: auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--fp8-append", action="store_true",
                   help="E4M3 workloads: the step also appends each sequence's new row\n"
                        "(E4M3 append policy, one more launch)")
    p.add_argument("--tile-ceiling", type=int, default=1, choices=(0, 1),
                   help="1: also time pkv_tile_read over the step's own tiles (its practical\n"
                        "read ceiling for this access pattern)")
    p.add_argument("--splits", type=int, default=16,
                   help="most pieces one sequence is cut into by the balanced split")
    p.add_argument("--n-query", type=int, default=1,
                   help="new tokens per sequence (speculative verify / chunked prefill; "
                        "balanced one-launch step only)")
    p.add_argument("--window", type=int, default=0,
                   help="sliding window in tokens (balanced one-launch step only; 0 = full)")
    p.add_argument("--unfused", action="store_true",
                   help="time append, decode and reduce as three launches")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget for the oracle baseline")
    p.add_argument("--op", default="step", choices=("step", "copy-blocks", "append-e4m3"),
                   help="step: the decode step (default); copy-blocks: the copy-on-write "
                        "block copy on the config's pools; append-e4m3: appending one token "
                        "per sequence into E4M3 blocks (use an E4M3 config, c5)")
    p.add_argument("--copy-pairs", type=int, default=2048,
                   help="block pairs per copy-blocks launch")
    p.add_argument("--steady-steps", type=int, default=2000,
                   help="after the timed passes, also time this many back-to-back steps after\n"
                        "--steady-warmup more (reported as steady_state, not as value; 0 = skip)")
    p.add_argument("--steady-warmup", type=int, default=500)
    p.add_argument("--read-ceiling-mib", type=int, default=1024,
                   help="after timing, read a buffer of this many MiB with the library's "
                        "streaming-read kernel and report the step's rate against it "
                        "(0 = skip)")
    p.add_argument("--paging-overhead", action="store_true",
                   help="also time the same steps with every sequence's blocks made "
                        "physically consecutive, and report the cost of paging itself")
    p.add_argument("--prefix", default="auto", choices=("auto", "no"),
                   help="auto: pass a shared prompt prefix (the prefix-shared config's 1024\n"
                        "tokens) to the step as prefix_blocks, read once per group of sequences\n"
                        "(attend, then a combine launch); no: the plain one-launch step with the\n"
                        "shared-blocks cache hint")
    p.add_argument("--shared-blocks", default="auto", choices=("auto", "yes", "no"),
                   help="pass the shared-blocks cache hint (auto: when the workload's tables "
                        "share a prefix)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="after timing, run plain device copies of this many MiB (a known-size "
                        "kernel that profiler byte counters can be scaled against)")
    return p.parse_args()


# --------------------------------------------------------------------------- CPU baseline
_CPU = {}


def _oracle_worker(seqs):
    from threadpoolctl import threadpool_limits

    from oracle import attn_ref

    d, cfg = _CPU["d"], _CPU["cfg"]
    with threadpool_limits(1):
        attn_ref(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                 cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"], seqs=seqs)
    return len(seqs)


def single_core(cfg, d, budget_s):
    """The oracle on one core (one thread): whole sequences of the batch in
    order (again from the first after the last) until about budget_s of
    work, at least one."""
    from threadpoolctl import threadpool_limits

    from oracle import attn_ref

    lens = d["context_lens"].astype(np.int64)
    done, tokens, t0 = 0, 0, time.perf_counter()
    with threadpool_limits(1):
        while done == 0 or time.perf_counter() - t0 < budget_s:
            b = done % cfg.B
            attn_ref(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                     cfg.scale, k_scale=d["k_scale"], v_scale=d["v_scale"], seqs=[b])
            tokens += int(lens[b])
            done += 1
    dt = time.perf_counter() - t0
    kv = synth.kv_bytes(cfg, [tokens])
    return {"config": cfg.name, "value": kv / dt / 1e9, "unit": "GB/s", "cores": 1,
            "sample": f"{done} sequences of the {cfg.B}-sequence batch in order, one thread",
            "seconds": dt, "step_seconds_extrapolated": dt * float(lens.sum()) / tokens}


def cpu_baseline(cfg, d, budget_s):
    """Time the fp64 oracle on a bounded sample of the batch, parallel over
    sequences with one single-threaded worker per host core of the box's
    share (fork, before the GPU is touched), and on one core for this
    config and the tiny config."""
    import multiprocessing as mp

    # the GPU machine allots 16 host cores to one GPU, whatever the affinity
    # mask shows: the pool never has more workers than that
    cores = min(len(os.sched_getaffinity(0)), 16)
    _CPU.update(d=d, cfg=cfg)
    lens = d["context_lens"].astype(np.int64)
    # probe one sequence to size the sample to the budget
    t0 = time.perf_counter()
    _oracle_worker([int(np.argmin(np.abs(lens - lens.mean())))])
    per_seq = max(time.perf_counter() - t0, 1e-4)
    n = int(max(1, min(cfg.B, budget_s * cores / per_seq)))
    seqs = list(range(n))
    chunks = [seqs[i::cores] for i in range(cores) if seqs[i::cores]]
    # when the sample is the whole batch and takes well under the budget,
    # repeat it so that the timing covers about budget_s of CPU work
    reps = max(1, int(budget_s / (per_seq * n)))
    ctx = mp.get_context("fork")
    with ctx.Pool(len(chunks)) as pool:
        pool.map(_oracle_worker, chunks)  # untimed: each worker's imports and first touches
        t0 = time.perf_counter()
        for _ in range(reps):
            pool.map(_oracle_worker, chunks)
        dt = (time.perf_counter() - t0) / reps
    kv = synth.kv_bytes(cfg, lens[:n])
    frac = float(lens[:n].sum() / lens.sum())
    return {
        "value": kv / dt / 1e9,
        "unit": "GB/s",
        "cores": len(chunks),
        "kind": "oracle",
        "sample": f"{n} of {cfg.B} sequences ({frac:.1%} of the step's KV tokens), "
                  f"{reps} pass(es), fp64 numpy, one single-threaded worker per core",
        "seconds": dt,
        "step_seconds_extrapolated": dt / frac,
        "cpu_model": _cpu_model(),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "single_core": [single_core(cfg, d, budget_s / 4)] + (
            [] if cfg.name == "c1" else
            [single_core(synth.CONFIGS["c1"], synth.generate(synth.CONFIGS["c1"]), 0.5)]),
    }


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# --------------------------------------------------------------------------- GPU run
def bench_copy_blocks(args, cfg, d):
    """Copy-on-write block copy: `--copy-pairs` whole blocks (K and V pools,
    all kv heads) per launch, two disjoint pair sets alternating."""
    import torch

    from paged_kv_cache_208_amd import _lib

    nb = d["nb"]
    n = min(args.copy_pairs, nb // 4)
    rng = np.random.default_rng(208_100)
    perm = rng.permutation(nb)
    sets = [(perm[0:n], perm[n:2 * n]), (perm[2 * n:3 * n], perm[3 * n:4 * n])]
    fp8 = cfg.kv_dtype == "e4m3"
    block_bytes = cfg.Hkv * 16 * cfg.D * (1 if fp8 else 2)
    moved = 2 * 2 * n * block_bytes + (2 * 2 * n * cfg.Hkv * 4 if fp8 else 0)  # read + write

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import copy_blocks_ref
        t0 = time.perf_counter()
        reps = 0
        while True:
            copy_blocks_ref(d["k_pool"], d["v_pool"], sets[reps % 2][0], sets[reps % 2][1],
                            d.get("k_scale"), d.get("v_scale"))
            reps += 1
            if time.perf_counter() - t0 > min(args.cpu_seconds, 5.0):
                break
        sec = (time.perf_counter() - t0) / reps
        cpu = {"value": moved / sec / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} full oracle calls ({n} pairs each, whole-pool copy-out "
                         "included), one core"}

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    kp, vp = up(d["k_pool"]), up(d["v_pool"])
    ks = up(d["k_scale"]) if fp8 else None
    vs = up(d["v_scale"]) if fp8 else None
    pairs = [(up(a.astype(np.int32)), up(b.astype(np.int32))) for a, b in sets]

    def launch(i):
        src, dst = pairs[i % 2]
        _lib.paged_kv_copy_blocks(kp, vp, src, dst, k_scale=ks, v_scale=vs, stream=stream)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(K):
        launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    value = moved / (ms * 1e-3) / 1e9
    achieved = moved / (k_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "copy-on-write block copy GB/s (HBM read + write)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8" if fp8 else "f16",
        "data": "synthetic",
        "config": {"workload": f"{n} block copies per launch on the pools of: {cfg.description}",
                   "name": cfg.name, "pairs": n, "block_bytes_per_pool": block_bytes},
        "kernel_us": round(k_ms * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_GBPS, 4), "traffic": None,
                     "kernel": "paged_kv_copy_blocks", "algorithmic_bytes_per_launch": moved},
        "cpu_baseline": cpu,
    }), flush=True)


def bench_append_e4m3(args, cfg, d):
    """One token per sequence appended into E4M3 blocks at each sequence's
    next position (sequences whose last block is full skip the step)."""
    import torch

    from paged_kv_cache_208_amd import _lib

    if cfg.kv_dtype != "e4m3":
        raise SystemExit("--op append-e4m3 needs an E4M3 config (c5)")
    rng = np.random.default_rng(208_200)
    B, Hkv, D = cfg.B, cfg.Hkv, cfg.D
    lens = d["context_lens"].astype(np.int64)
    tab = d["block_tables"]
    slots = np.array([int(tab[b, L // 16]) * 16 + L % 16 if L % 16 else -1
                      for b, L in enumerate(lens)], dtype=np.int64)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    live = int((slots >= 0).sum())
    # algorithmic bytes when no row is re-encoded: new rows in (fp16), codes out, scales
    moved = live * Hkv * 2 * (D * 2 + D + 8)

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    g = {k: up(v) for k, v in (("kp", d["k_pool"]), ("vp", d["v_pool"]), ("ks", d["k_scale"]),
                               ("vs", d["v_scale"]), ("kn", kn), ("vn", vn), ("sl", slots))}

    def launch():
        _lib.paged_kv_append_e4m3(g["kn"], g["vn"], g["kp"], g["vp"], g["ks"], g["vs"], g["sl"],
                                  stream=stream)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(K):
        launch()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    print(json.dumps({
        "metric": "E4M3 append latency per step (us) and GB/s",
        "value": round(ms * 1e3, 3), "unit": "us", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"one token per sequence ({live} of {B}) into the E4M3 pools of: "
                               f"{cfg.description}", "name": cfg.name},
        "gbps": round(moved / (ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "latency", "achieved": round(moved / (ms * 1e-3) / 1e9, 2),
                     "peak": HBM_GBPS, "unit": "GB/s",
                     "frac": round(moved / (ms * 1e-3) / 1e9 / HBM_GBPS, 5), "traffic": None,
                     "kernel": "paged_kv_append_e4m3", "algorithmic_bytes_per_launch": moved},
        "cpu_baseline": None,
    }), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sequences and kv heads shard across GPUs with no exchange; see the design "
              "notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    cfg = synth.CONFIGS[args.config]
    if args.partition_size is not None:
        cfg = cfg.replace(partition_size=args.partition_size)
    t0 = time.perf_counter()
    d = synth.generate(cfg)
    print(f"# generated {cfg.name} in {time.perf_counter() - t0:.1f}s: B={cfg.B} "
          f"Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} kv={cfg.kv_dtype} PS={cfg.partition_size} "
          f"NB={d['nb']}", file=sys.stderr, flush=True)

    if args.op == "copy-blocks":
        bench_copy_blocks(args, cfg, d)
        return
    if args.op == "append-e4m3":
        bench_append_e4m3(args, cfg, d)
        return

    if args.fp8_append and cfg.kv_dtype == "e4m3" and d.get("k_new") is None:
        # the new rows the E4M3 step appends (fp16 N(0, 1), a seeded draw of
        # their own)
        rng = np.random.default_rng(208_900)
        d = dict(d, k_new=rng.standard_normal((cfg.B, cfg.Hkv, cfg.D)).astype(np.float16),
                 v_new=rng.standard_normal((cfg.B, cfg.Hkv, cfg.D)).astype(np.float16))
    nq = args.n_query
    # a chunk wider than one 16-column product (g * nq > 16) is appended by
    # paged_kv_append (one slot per new token, QK-norm + RoPE at each token's
    # position for the fused config) and then attended by the step
    chunk = nq > 1 and cfg.group * nq > 16
    if nq > 1:
        # several new tokens per sequence: q and the new rows get a token axis
        rng = np.random.default_rng(208_300)
        d = dict(d, q=rng.standard_normal((cfg.B, nq, cfg.Hq, cfg.D)).astype(np.float16),
                 k_new=rng.standard_normal((cfg.B, nq, cfg.Hkv, cfg.D)).astype(np.float16),
                 v_new=rng.standard_normal((cfg.B, nq, cfg.Hkv, cfg.D)).astype(np.float16))
        if chunk:
            lens = d["context_lens"].astype(np.int64)
            if int(lens.min()) < nq:
                sys.exit(f"--n-query {nq} needs every context to hold the chunk (min L {lens.min()})")
            tok = np.array([[L - nq + j + 1 for j in range(nq)] for L in lens], dtype=np.int32)
            tab, BS = d["block_tables"], cfg.block_size
            d["chunk_slots"] = np.array([[int(tab[b, (p - 1) // BS]) * BS + (p - 1) % BS
                                          for p in tok[b]] for b in range(cfg.B)],
                                        dtype=np.int64).reshape(-1)
            d["chunk_lens"] = tok.reshape(-1)
        args.no_cpu_baseline = True

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, d, args.cpu_seconds)
        print(f"# cpu baseline: {cpu['value']:.3f} GB/s on {cpu['cores']} cores "
              f"({cpu['seconds']:.1f}s)", file=sys.stderr, flush=True)

    import torch

    from paged_kv_cache_208_amd import _lib

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    def up(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    base = {k: up(v) for k, v in d.items() if isinstance(v, np.ndarray)}
    footprint = sum(t.numel() * t.element_size() for t in base.values())
    R = args.rotate or max(2, math.ceil(ROTATE_BYTES / footprint))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    B, Hq, D = d["q"].shape[0], d["q"].shape[-2], d["q"].shape[-1]
    PS = cfg.partition_size
    P = _lib.max_partitions_for(cfg.mbs, PS)
    ws = _lib.alloc_partials(B, Hq, D, P, dev) if PS else None
    # the one-launch step splits contexts evenly over all waves (partition_size 0)
    # unless --partition-size asks for fixed partitions
    step_ps = PS if args.partition_size is not None else 0
    step_ws = _lib.alloc_step_workspace(B, Hq * nq, cfg.Hkv, D, P if step_ps else args.splits,
                                        dev)
    out = torch.empty(tuple(d["q"].shape), dtype=torch.float16, device=dev)
    fp8 = cfg.kv_dtype == "e4m3"
    torch.cuda.synchronize()

    ev = {}

    # the caller's block manager knows when tables share blocks (reference
    # counts); the hint only picks the KV loads' cache policy
    shared = (cfg.prefix_tokens > 0) if args.shared_blocks == "auto" else args.shared_blocks == "yes"
    # the caller's block manager knows the shared prefix; the step then reads
    # each prefix tile once per group of sequences
    prefix_blocks = (cfg.prefix_tokens // cfg.block_size
                     if args.prefix == "auto" and cfg.prefix_tokens and not args.unfused and nq == 1
                     and not args.window and args.partition_size is None else 0)
    if prefix_blocks and args.shared_blocks == "auto":
        shared = False  # the prefix step picks the cache policy per tile itself

    def step_unfused(g, i, timed):
        if not fp8:
            kw = {}
            if cfg.fused_append:
                kw = dict(q=g["q"], gamma_q=g["gamma_q"], gamma_k=g["gamma_k"],
                          context_lens=g["context_lens"], eps=cfg.eps, rope_theta=cfg.theta)
            _lib.paged_kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"],
                                 g["slot_mapping"], stream=stream, **kw)
        if timed:
            ev["d0"][i].record(stream)
        _lib.paged_attn_decode(out if PS == 0 else None, g["q"], g["k_pool"], g["v_pool"],
                               g["block_tables"], g["context_lens"], cfg.scale,
                               k_scale=g.get("k_scale"), v_scale=g.get("v_scale"),
                               partition_size=PS, part_out=ws and ws[0],
                               part_max=ws and ws[1], part_sum=ws and ws[2],
                               shared_blocks=shared, stream=stream)
        if timed:
            ev["d1"][i].record(stream)
        if PS:
            _lib.paged_attn_reduce(out, ws[0], ws[1], ws[2], g["context_lens"], PS,
                                   stream=stream)

    def decode_only(g):
        _lib.paged_attn_decode(out if PS == 0 else None, g["q"], g["k_pool"], g["v_pool"],
                               g["block_tables"], g["context_lens"], cfg.scale,
                               k_scale=g.get("k_scale"), v_scale=g.get("v_scale"),
                               partition_size=PS, part_out=ws and ws[0],
                               part_max=ws and ws[1], part_sum=ws and ws[2],
                               shared_blocks=shared, stream=stream)

    def step_fused(g, i, timed):
        kw = {}
        if not fp8 or args.fp8_append:
            kw = dict(k_new=g["k_new"], v_new=g["v_new"])
            if cfg.fused_append:
                kw.update(gamma_q=g["gamma_q"], gamma_k=g["gamma_k"], eps=cfg.eps,
                          rope_theta=cfg.theta)
        if timed:
            ev["d0"][i].record(stream)
        if chunk:
            # the chunk's rows go in first (one launch), then the step attends
            B_, Hkv_ = g["k_new"].shape[0], g["k_new"].shape[2]
            akw = {}
            if cfg.fused_append:
                akw = dict(q=g["q"].view(B_ * nq, cfg.Hq, cfg.D), gamma_q=g["gamma_q"],
                           gamma_k=g["gamma_k"], context_lens=g["chunk_lens"], eps=cfg.eps,
                           rope_theta=cfg.theta)
            if not fp8:
                _lib.paged_kv_append(g["k_new"].view(B_ * nq, Hkv_, cfg.D),
                                     g["v_new"].view(B_ * nq, Hkv_, cfg.D), g["k_pool"],
                                     g["v_pool"], g["chunk_slots"], stream=stream, **akw)
            kw = {}
        _lib.paged_decode_step(out, g["q"], g["k_pool"], g["v_pool"], g["block_tables"],
                               g["context_lens"], cfg.scale, k_scale=g.get("k_scale"),
                               v_scale=g.get("v_scale"), partition_size=step_ps,
                               window=args.window, prefix_blocks=prefix_blocks,
                               workspace=step_ws, shared_blocks=shared, stream=stream, **kw)
        if timed:
            ev["d1"][i].record(stream)

    def step(i, timed=False):
        g = copies[i % R]
        (step_unfused if args.unfused else step_fused)(g, i, timed)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # pass 1: the K steps back to back, one event pair around all of them
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    # pass 2: the same K steps with an event pair around each decode launch
    # (the pairs add a little time between launches, so pass 1 gives the rate)
    ev["d0"] = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev["d1"] = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        step(i, timed=True)
    torch.cuda.synchronize()
    dec_ms = [ev["d0"][i].elapsed_time(ev["d1"][i]) for i in range(K)]
    dec_avg = float(np.mean(dec_ms))
    # pass 3 (several launches per step): the decode launch alone, K times back
    # to back, which times that kernel without the event pairs' own cost
    dec_b2b = None
    if args.unfused:
        for i in range(args.warmup):
            decode_only(copies[i % R])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            decode_only(copies[i % R])
        e1.record(stream)
        torch.cuda.synchronize()
        dec_b2b = e0.elapsed_time(e1) / K

    def back_to_back():
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for i in range(K):
            step(i)
        s1.record(stream)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / K

    # steady state: a longer run after the timed passes (the first ~10-30 ms
    # of sustained work after the process starts run slower, and a short
    # window also carries its first launch's host latency); reported beside
    # `value`, which stays the W / K window's
    steady_ms = None
    if args.steady_steps > 0:
        for i in range(args.steady_warmup):
            step(i)
        torch.cuda.synchronize()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record(stream)
        for i in range(args.steady_steps):
            step(i)
        q1.record(stream)
        torch.cuda.synchronize()
        steady_ms = q0.elapsed_time(q1) / args.steady_steps

    # the step's practical read ceiling: its tiles, in its order and split,
    # read with its cache policies and nothing computed (pkv_tile_read)
    tile_ms = None
    if args.tile_ceiling and not args.unfused and step_ps == 0 and not args.window:
        ids = torch.from_numpy(step_tile_ids(cfg, d, nq, prefix_blocks, shared)).to(dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        waves = cus * 4 * (2 if fp8 else 1)

        def tile_read(i):
            g = copies[i % R]
            _lib.pkv_tile_read(g["k_pool"], g["v_pool"], ids, waves, sink, stream=stream)

        for i in range(args.warmup):
            tile_read(i)
        torch.cuda.synchronize()
        t0e, t1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0e.record(stream)
        for i in range(K):
            tile_read(i)
        t1e.record(stream)
        torch.cuda.synchronize()
        tile_ms = t0e.elapsed_time(t1e) / K
        del ids, sink

    paging = None
    if args.paging_overhead:
        # the same batch with each sequence's blocks made consecutive
        del copies[:]
        torch.cuda.synchronize()
        d2 = synth.contiguous_layout(cfg, d)
        base2 = {k: up(v) for k, v in d2.items() if isinstance(v, np.ndarray)}
        copies.extend([base2] + [{k: v.clone() for k, v in base2.items()} for _ in range(R - 1)])
        ms_contig = back_to_back()
        paging = {"ms_per_step_contiguous": round(ms_contig, 5),
                  "overhead_pct": round(100.0 * (ms / ms_contig - 1.0), 2)}
        del copies[:], base2, d2
        torch.cuda.synchronize()

    ceiling = None
    if args.read_ceiling_mib:
        nbytes = args.read_ceiling_mib << 20
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            _lib.pkv_stream_read(buf, sink, stream=stream)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record(stream)
        for _ in range(10):
            _lib.pkv_stream_read(buf, sink, stream=stream)
        c1.record(stream)
        torch.cuda.synchronize()
        ceiling = nbytes / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
        del buf, sink

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    kv = synth.kv_bytes(cfg, d["context_lens"], args.window)
    # distinct blocks' bytes (a shared prefix once): what HBM must deliver at
    # least, so the fraction of peak is priced on it; kv (logical) gives the
    # effective rate the attention sees
    kv_unique = synth.unique_kv_bytes(cfg, d["context_lens"]) if not args.window else kv
    tokens = int(d["context_lens"].astype(np.int64).sum())
    traffic = None
    fused_balanced = (not args.unfused and step_ps == 0 and args.splits == 16 and not args.window
                      and nq == 1 and not args.fp8_append)
    measured = (MEASURED_TRAFFIC.get((cfg.name, step_source_hash(prefix=prefix_blocks > 0), shared,
                                      prefix_blocks))
                if fused_balanced else None)
    if measured:
        traffic = measured["fetch_bytes"] + measured["write_bytes"]
    value = kv / (ms * 1e-3) / 1e9
    # the kernel's average launch duration: with one launch per step, the
    # back-to-back pass times exactly the step kernel's launches (rocprof's
    # average duration agrees to ~0.2%), while pass 2's event pair around
    # every launch adds ~2.5 us of its own; with several launches per step
    # (--unfused) pass 3 times the decode kernel alone, back to back
    one_launch = not args.unfused
    kernel_ms = min(ms, dec_avg) if one_launch else dec_b2b
    achieved = kv_unique / (kernel_ms * 1e-3) / 1e9
    unique_rate = kv_unique / (ms * 1e-3) / 1e9
    # launches per step: the unfused path's append, decode and reduce; the
    # one-launch fixed partitions; the balanced split's attend and combine
    # (one launch with QK-norm inside the step); a chunk's append before it
    if args.unfused:
        launches = (3 if not fp8 else 2) if PS else (2 if not fp8 else 1)
    elif step_ps:
        launches = 1
    else:
        launches = ((1 if cfg.fused_append and not chunk else 2) + (1 if chunk and not fp8 else 0)
                    + (1 if fp8 and args.fp8_append else 0))
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3-kv/f16-q/f32-acc" if fp8 else "f16-kv/f32-acc",
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "name": cfg.name,
            "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "head_dim": cfg.D, "block_size": 16,
            "kv_dtype": cfg.kv_dtype,
            "split": (f"fixed {PS}-token partitions" if args.unfused or step_ps
                      else f"balanced over all waves, <= {args.splits} pieces per sequence"),
            "context_tokens": tokens, "mean_context": round(tokens / cfg.B, 1),
            "step": (("append+attend+combine" if args.fp8_append else "attend+combine") if fp8 else
                     ("qknorm_rope+append+attend+combine" if cfg.fused_append
                      else "append+attend+combine")),
            "launches_per_step": launches,
            "window": args.window,
            "new_tokens_per_sequence": nq,
            "shared_prefix_blocks": prefix_blocks,
            "rotated_copies": R,
            "kv_load_policy": "cached (shared-blocks hint)" if shared else "non-temporal",
        },
        "steps_per_s": round(1e3 / ms, 1),
        "tokens_per_s": round(cfg.B * nq * 1e3 / ms, 1),
        "pct_hbm_peak": round(100 * unique_rate / HBM_GBPS, 2),
        "read_ceiling_gbps": None if ceiling is None else round(ceiling, 1),
        "pct_of_read_ceiling": None if ceiling is None else round(100 * unique_rate / ceiling, 2),
        "tile_read_us": None if tile_ms is None else round(tile_ms * 1e3, 3),
        "tile_read_ceiling_gbps": (None if tile_ms is None
                                   else round(kv_unique / (tile_ms * 1e-3) / 1e9, 1)),
        "pct_of_tile_read_ceiling": (None if tile_ms is None
                                     else round(100 * tile_ms / kernel_ms, 2)),
        "paging": paging,
        "steady_state": None if steady_ms is None else {
            "warmup": args.steady_warmup, "steps": args.steady_steps,
            "ms_per_step": round(steady_ms, 5),
            "unique_kv_gbps": round(kv_unique / (steady_ms * 1e-3) / 1e9, 2),
            "frac_of_hbm_peak": round(kv_unique / (steady_ms * 1e-3) / 1e9 / HBM_GBPS, 4)},
        "kv_bytes_per_step": kv,
        "unique_kv_bytes_per_step": kv_unique,
        "unique_kv_gbps": round(unique_rate, 2),
        "decode_kernel_us": round(dec_avg * 1e3, 3),
        "kernel_us_for_roofline": round(kernel_ms * 1e3, 3),
        "decode_only_us_back_to_back": round(dec_b2b * 1e3, 3) if dec_b2b else None,
        "decode_kernel_us_p10_p50_p90": [round(float(np.percentile(dec_ms, q)) * 1e3, 2)
                                         for q in (10, 50, 90)],
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_GBPS, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per launch (HBM read + write)",
            "traffic_detail": measured,
            "kernel": "paged_attn_decode" if args.unfused else "paged_decode_step",
            "algorithmic_bytes_per_launch": kv_unique,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
