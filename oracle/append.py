"""KV append and the Qwen3 QK-norm + split-half RoPE prologue (oracle side).

Append (scatter)
----------------
"Distributed LLM Inference Serving Platform", section 5.1: prompt K/V are
written directly into the physical blocks assigned to the request, and each
decode step allocates one more token page when the tail block is full.  The
library receives the destination of every new token as a flat slot index
    slot = physical_block * BS + offset_in_block
(slot < 0: the token is skipped), so the write for token i is
    k_pool[slot // BS, :, slot % BS, :] = k_new[i]      (same for v)
Nothing else in the pools changes.

QK-norm + split-half RoPE
-------------------------
"Roadmap: vLLM-style serving features for TornadoVM batched decode",
Core batched decode: Qwen3 decoding uses a per-head QK-norm followed by a
split-half RoPE; the Mistral comment makes the RoPE base theta a model
parameter.  The pages give no formulas; the readings taken are the standard
ones:
  * RMSNorm over head_dim for every q and k head:
        r = x / sqrt(mean(x^2) + eps) * gamma          (gamma shared by heads)
  * split-half rotation at position pos = context_len - 1 (the new token is
    the last of the L tokens), pairing element i with element i + D/2:
        f_i = theta^(-2i/D),   a = pos * f_i
        y_i       = r_i cos a - r_{i+D/2} sin a
        y_{i+D/2} = r_{i+D/2} cos a + r_i sin a
  * v is copied unchanged.
All of it is evaluated in float64 and rounded once to float16
(round-to-nearest-even) for storage.

Pins (tests/test_rope_norm.py, tests/test_append_oracle.py): mpmath 50-digit
brute force at positions 0, 1 and 8191; RMS of the normalised vector with
gamma = 1; identity rotation at position 0; per-pair norm preservation;
relative-position property of the rotated dot product; a hand-written
scatter fixture (tests/golden/append_scatter.json).
"""

import numpy as np


def append_ref(k_pool, v_pool, k_new, v_new, slot_mapping, block_size=16):
    """Return new (k_pool, v_pool) copies with token rows scattered in."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, off = int(slot) // block_size, int(slot) % block_size
        k_out[blk, :, off, :] = k_new[i]
        v_out[blk, :, off, :] = v_new[i]
    return k_out, v_out


def rmsnorm_rope_ref(x, gamma, pos, eps, theta):
    """float64 [T, H, D]: per-head RMSNorm (gamma) then split-half RoPE.

    x: [T, H, D] float16, gamma: [D], pos: [T] integer positions.
    """
    xf = np.asarray(x, dtype=np.float64)
    T, H, D = xf.shape
    half = D // 2
    ms = np.mean(xf * xf, axis=-1, keepdims=True)
    r = xf / np.sqrt(ms + float(eps)) * np.asarray(gamma, dtype=np.float64)
    i = np.arange(half, dtype=np.float64)
    freq = np.power(float(theta), -2.0 * i / D)                  # [half]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :]  # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    lo, hi = r[..., :half], r[..., half:]
    y = np.empty_like(r)
    y[..., :half] = lo * c - hi * s
    y[..., half:] = hi * c + lo * s
    return y


def fused_append_ref(q, k_new, v_new, k_pool, v_pool, slot_mapping, context_lens,
                     gamma_q, gamma_k, eps, theta, block_size=16):
    """Qwen3 decode prologue + append.

    Returns (q_out fp16 [T,Hq,D], k_pool', v_pool', q_exact f64, k_exact f64):
    q and k are normalised and rotated at pos = context_lens[i] - 1 and
    rounded once to fp16; k' and v are then scattered like append_ref.
    """
    pos = np.asarray(context_lens, dtype=np.int64) - 1
    q_exact = rmsnorm_rope_ref(q, gamma_q, pos, eps, theta)
    k_exact = rmsnorm_rope_ref(k_new, gamma_k, pos, eps, theta)
    q_out = q_exact.astype(np.float16)
    k_rot = k_exact.astype(np.float16)
    kp, vp = append_ref(k_pool, v_pool, k_rot, v_new, slot_mapping, block_size)
    return q_out, kp, vp, q_exact, k_exact
