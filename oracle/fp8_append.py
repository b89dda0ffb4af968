"""Appending a new token into an E4M3 KV block with per-(block, kv head)
scales (oracle side).

"Roadmap: vLLM-style serving features for TornadoVM batched decode",
Sampling / logits, lists a quantized (Q8/FP8) KV cache; the pages fix no
quantisation policy.  The reading taken here keeps every block's scale at
the running amax of the rows written so far, divided by the format's
largest value:

    s = max |value| over the block's rows (this kv head) / 448

For token i with slot p = slot_mapping[i] >= 0, block n = p // 16,
row r = p % 16, and for K and V of every kv head separately:
  1. x = the new row (fp16, exact in float32); a = max |x|.
  2. s_old = scale[n][h] if r > 0, else 0 (a block starts empty).
  3. If a > 448 * s_old: s_new = a / 448, and rows 0..r-1 are re-encoded
        c' = enc( (dec(c) * s_old) / s_new )
     (when s_old is 0 they are all zero and stay so); else s_new = s_old.
  4. Row r = enc(x / s_new) (0 when s_new is 0); scale[n][h] = s_new.
Every arithmetic step is a float32 operation in the order written (the
kernel's precision: the code is an integer decided by float arithmetic, so
both sides decide it the same way); enc is round-to-nearest-even with the
magnitude clamped to 448 (oracle/e4m3.py).  Rows past r are not touched.

Pins (tests/test_fp8_append_oracle.py): the scale equals the float32 amax
of all rows written to the block over 448 after every append; rows are not
re-encoded when the amax does not grow; each stored value is within half an
E4M3 spacing (relative 2^-4, absolute 2^-10 * s below the normal range) of
its exact value, and within two such roundings after a re-encoding; a row of
equal magnitudes decodes to exactly +-448 * s; a new block ignores stale
bytes in its other rows.
"""

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_encode, e4m3_table

F32 = np.float32


def _quantize_row(x32, s):
    if s == F32(0):
        return np.zeros(x32.shape, dtype=np.uint8)
    return e4m3_encode((x32 / s).astype(F32))


def append_e4m3_ref(k_pool, v_pool, k_scale, v_scale, k_new, v_new, slot_mapping,
                    block_size=16):
    """Returns (k_pool', v_pool', k_scale', v_scale') after appending every
    token with slot >= 0, in token order (slots of one call lie in distinct
    blocks)."""
    pools = [np.array(k_pool, copy=True), np.array(v_pool, copy=True)]
    scales = [np.array(k_scale, dtype=F32, copy=True), np.array(v_scale, dtype=F32, copy=True)]
    news = [np.asarray(k_new), np.asarray(v_new)]
    table = e4m3_table()
    for i, p in enumerate(np.asarray(slot_mapping).reshape(-1)):
        p = int(p)
        if p < 0:
            continue
        n, r = p // block_size, p % block_size
        for pool, scale, new in zip(pools, scales, news):
            for h in range(pool.shape[1]):
                x = new[i, h].astype(F32)
                a = F32(np.max(np.abs(x)))
                s_old = scale[n, h] if r > 0 else F32(0)
                if a > F32(E4M3_MAX) * s_old:
                    s_new = F32(a / F32(E4M3_MAX))
                    if r > 0 and s_old != F32(0):
                        old = table[pool[n, h, :r]].astype(F32)      # exact
                        v = ((old * s_old).astype(F32) / s_new).astype(F32)
                        pool[n, h, :r] = e4m3_encode(v)
                else:
                    s_new = s_old
                pool[n, h, r] = _quantize_row(x, s_new)
                scale[n, h] = s_new
    return pools[0], pools[1], scales[0], scales[1]
