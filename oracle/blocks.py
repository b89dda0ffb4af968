"""Copy-on-write block copy (oracle side).

"Distributed LLM Inference Serving Platform", section 11, worked solution of
Lab 1 (copy-on-write for parallel sampling), and section 7 (block manager):
when a sequence appends into a tail block that other sequences still share,
it takes a fresh physical block, the tokens already in the shared block are
copied into it, and the sequence's table points at the copy from then on.
The copy itself is plain data movement: for every pair (src, dst)

    k_pool[dst] = k_pool[src]        (all kv heads, all BS rows)
    v_pool[dst] = v_pool[src]
    k_scale[dst] = k_scale[src], v_scale[dst] = v_scale[src]   (E4M3 pools)

Reading taken here: whole blocks are copied (rows past the copied tokens are
never read, because context lengths bound every read); the destinations are
distinct and none of them is also a source, so the order of the pairs does
not matter; every other block is left as it was.

Pins (tests/test_blocks_oracle.py): the Lab 1 worked example driven through
the host block manager (pool.py) gives every child, read through its own
table, exactly the parent's tokens; untouched blocks compare bitwise; the
copies equal their sources bitwise, for fp16 and E4M3 pools with scales.
"""

import numpy as np


def copy_blocks_ref(k_pool, v_pool, src, dst, k_scale=None, v_scale=None):
    """Returns copies of the pools (and scales, when given) after the copy."""
    src = [int(s) for s in np.asarray(src).reshape(-1)]
    dst = [int(d) for d in np.asarray(dst).reshape(-1)]
    if len(src) != len(dst):
        raise ValueError("src and dst differ in length")
    if len(set(dst)) != len(dst) or set(dst) & set(src):
        raise ValueError("destinations must be distinct and must not be sources")
    kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    ks = None if k_scale is None else np.array(k_scale, copy=True)
    vs = None if v_scale is None else np.array(v_scale, copy=True)
    for s, d in zip(src, dst):
        kp[d] = k_pool[s]
        vp[d] = v_pool[s]
        if ks is not None:
            ks[d] = k_scale[s]
            vs[d] = v_scale[s]
    return kp, vp, ks, vs
