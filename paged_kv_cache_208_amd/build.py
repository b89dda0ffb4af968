"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_208_amd.build

compiles every HIP source under csrc/ plus the host-only argument checks
into paged_kv_cache_208_amd/libpagedkv.so.  hipcc cross-compiles for gfx950,
so this runs on machines without a GPU.
"""

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpagedkv.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms stay off: the compiler would otherwise form
# v_pk_{add,mul,fma}_f32 from scalar float code.
# -amdgpu-kernarg-preload-count: the first three kernel arguments arrive in
# SGPRs at dispatch (the step kernels put the lengths pointer, the batch size
# and the wave count there, so their first load needs no load of the
# argument block); a kernel whose first argument is a struct preloads nothing.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-kernarg-preload-count=3"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "validate.cpp")]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag: harmless
    err = "\n".join(ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln)
    return res.returncode, err


def build(out=LIB, extra=(), verbose=False, jobs=None):
    """Compile each source to an object in parallel, then link the library."""
    common = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              *DEVICE_FLAGS, *extra]
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="pagedkv_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        cmds = [common + ["-c", "-o", o, s] for s, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            results = list(pool.map(_run, cmds))
        for (rc, err), s in zip(results, srcs):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        link = [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", out + ".tmp", *objs]
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
