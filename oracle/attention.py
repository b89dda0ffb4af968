"""Batched-decode paged attention, float64 reference (oracle side).

Definition followed
-------------------
"Distributed LLM Inference Serving Platform", section 2 (Mental Model and
Architectural Abstraction): a sequence's KV cache is cut into fixed 16-token
logical blocks; the block table maps logical block n (tokens 16n .. 16n+15)
to a physical block anywhere in the pool.  Paging is address translation, so
the result is ordinary attention over the sequence's contiguous K/V.
Section 5.1 (request lifecycle): in a decode step each sequence submits one
token, which attends over all blocks in its own table.  Section 3
(terminology) calls PagedAttention the attention kernel that reads K/V from
non-contiguous physical blocks through page tables.

Grouped-query attention: section 1 names 8:1 GQA; the head mapping is not
printed, and the reading taken is the contiguous grouping q head h -> kv head
h // (Hq / Hkv).

So for sequence b with L = context_lens[b] valid tokens (positions 0..L-1),
q head h and kv head j = h // g:
    s_t = scale * <q[b,h], K_b[j,t]>,   t = 0..L-1
    out[b,h] = sum_t softmax(s)_t * V_b[j,t]
computed here in float64 with the textbook max-subtracted softmax.  The
online softmax, the split into partitions and the block tiling the GPU uses
are NOT modelled: they reach this same value up to rounding.

Layouts (the pages fix none; chosen for the library and mirrored here):
    q            [B, Hq, D]               float16
    k/v pool     [NB, Hkv, BS, D]         float16, or uint8 E4M3 codes
    k/v scale    [NB, Hkv]                float32, E4M3 only: real = code*scale
    block_tables [B, MBS]                 int32
    context_lens [B]                      int32

Pins (tests/test_oracle.py): Decimal 50-digit brute force on tiny inputs,
closed forms (L = 1, q = 0, constant V, one dominant key), softmax weights
summing to one, identity table == permuted table, GQA == MHA with repeated
KV heads, partials + combine == unsplit.
"""

import numpy as np

from .e4m3 import e4m3_decode


def gather_sequence_kv(pool, scales, table_row, L, block_size):
    """Contiguous float64 [Hkv, L, D] view of one sequence's K (or V).

    The first ceil(L / block_size) entries of the table row are the physical
    blocks holding tokens 0..L-1 in order (logical block n holds tokens
    n*BS .. n*BS+BS-1).  Entries after those are never read.
    """
    n = -(-L // block_size)
    ids = np.asarray(table_row[:n], dtype=np.int64)
    blocks = pool[ids]                                    # [n, Hkv, BS, D]
    if pool.dtype == np.uint8:
        vals = e4m3_decode(blocks)
        vals = vals * np.asarray(scales, dtype=np.float64)[ids][:, :, None, None]
    else:
        vals = blocks.astype(np.float64)
    hkv, d = vals.shape[1], vals.shape[3]
    seq = vals.transpose(1, 0, 2, 3).reshape(hkv, n * block_size, d)
    return seq[:, :L, :]


def _softmax(s):
    m = np.max(s)
    w = np.exp(s - m)
    return w / np.sum(w)


def attn_weights_ref(q, k_pool, block_tables, context_lens, scale, *,
                     k_scale=None, block_size=16):
    """Softmax weights p[b][h] (float64 [L_b]) as a list of lists."""
    B, Hq, _ = q.shape
    Hkv = k_pool.shape[1]
    g = Hq // Hkv
    out = []
    for b in range(B):
        L = int(context_lens[b])
        row = []
        if L > 0:
            K = gather_sequence_kv(k_pool, k_scale, block_tables[b], L, block_size)
        for h in range(Hq):
            if L == 0:
                row.append(np.zeros(0))
                continue
            qh = q[b, h].astype(np.float64)
            s = float(scale) * (K[h // g] @ qh)
            row.append(_softmax(s))
        out.append(row)
    return out


def attn_ref(q, k_pool, v_pool, block_tables, context_lens, scale, *,
             k_scale=None, v_scale=None, block_size=16, seqs=None, window=0):
    """float64 [B, Hq, D] attention output (unrounded).

    L_b = 0 gives a zero row (no tokens to attend over; this library's
    convention, the pages never reach that case).  ``seqs`` restricts the
    work to the listed sequences; other rows are left NaN.

    window > 0: sliding-window attention ("Roadmap: vLLM-style serving
    features for TornadoVM batched decode", Models: the Gemma 4 batched
    decode has sliding-window layers; the pages give no detail).  Reading
    taken: the query at position L_b - 1 attends to the last ``window``
    tokens, positions max(0, L_b - window) .. L_b - 1; window = 0 is full
    attention.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(context_lens[b])
        if L == 0:
            out[b] = 0.0
            continue
        K = gather_sequence_kv(k_pool, k_scale, block_tables[b], L, block_size)
        V = gather_sequence_kv(v_pool, v_scale, block_tables[b], L, block_size)
        if window > 0 and L > window:
            K, V = K[:, L - window:], V[:, L - window:]
        for h in range(Hq):
            j = h // g
            s = float(scale) * (K[j] @ q[b, h].astype(np.float64))
            p = _softmax(s)
            out[b, h] = p @ V[j]
    return out


def partials_ref(q, k_pool, v_pool, block_tables, context_lens, scale,
                 partition_size, *, k_scale=None, v_scale=None, block_size=16):
    """Per-partition softmax statistics, float64.

    Partition p of sequence b covers tokens [p*PS, min(L_b, (p+1)*PS)); there
    are P_b = ceil(L_b / PS) of them.  For each (b, h, p):
        m = max_t s_t,  l = sum_t exp(s_t - m),  o = sum_t exp(s_t - m) V_t / l
    with s in natural-log units (s = scale * q.k).  Returns (m, l, o) shaped
    [B, Hq, Pmax], [B, Hq, Pmax], [B, Hq, Pmax, D]; slots p >= P_b are NaN.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    g = Hq // Hkv
    PS = int(partition_size)
    pmax = max([-(-int(L) // PS) for L in context_lens] + [1])
    m = np.full((B, Hq, pmax), np.nan)
    l = np.full((B, Hq, pmax), np.nan)
    o = np.full((B, Hq, pmax, D), np.nan)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = gather_sequence_kv(k_pool, k_scale, block_tables[b], L, block_size)
        V = gather_sequence_kv(v_pool, v_scale, block_tables[b], L, block_size)
        for h in range(Hq):
            j = h // g
            s = float(scale) * (K[j] @ q[b, h].astype(np.float64))
            for p in range(-(-L // PS)):
                lo, hi = p * PS, min(L, (p + 1) * PS)
                sp = s[lo:hi]
                mp = np.max(sp)
                w = np.exp(sp - mp)
                m[b, h, p] = mp
                l[b, h, p] = np.sum(w)
                o[b, h, p] = (w @ V[j, lo:hi]) / l[b, h, p]
    return m, l, o


def combine_ref(m, l, o, context_lens, partition_size):
    """Combine per-partition (m, l, o) into the full softmax output.

    With M = max_p m_p and w_p = l_p * exp(m_p - M):
        out = sum_p w_p o_p / sum_p w_p      over p < ceil(L_b / PS).
    Each partition's o_p is its own normalised average, so weighting it by
    its share of the total softmax mass recovers the unsplit result exactly
    (up to rounding).  L_b = 0 gives a zero row.
    """
    B, Hq, _, D = o.shape
    PS = int(partition_size)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        P = -(-int(context_lens[b]) // PS)
        if P == 0:
            continue
        for h in range(Hq):
            mp = m[b, h, :P]
            M = np.max(mp)
            w = l[b, h, :P] * np.exp(mp - M)
            out[b, h] = (w @ o[b, h, :P]) / np.sum(w)
    return out


def mq_attn_ref(q, k_pool, v_pool, block_tables, context_lens, scale, *,
                k_scale=None, v_scale=None, block_size=16):
    """Several new query tokens per sequence with a causal mask, float64.

    "Roadmap: vLLM-style serving features for TornadoVM batched decode",
    Deferred / WIP: speculative decoding verifies a batch of drafted tokens in
    one forward (1.71 tokens per forward), and chunked prefill would put
    several tokens of a sequence in one step.  Reading taken: q is
    [B, nq, Hq, D]; context_lens[b] = L counts the nq new tokens, which sit
    at positions L - nq .. L - 1; new token j attends to positions
    0 .. L - nq + j (itself and everything before it):
        s_t = scale * <q[b, j, h], K_b[h // g, t]>   for t <= L - nq + j,
        out[b, j, h] = sum_t softmax(s)_t V_b[h // g, t]
    The mask is written out on the full score vector (masked scores are
    -inf before the softmax).  L = 0 gives zero rows; 0 < L < nq is outside
    the contract.
    """
    B, nq, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, nq, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        if L < nq:
            raise ValueError("each sequence must hold its nq new tokens")
        K = gather_sequence_kv(k_pool, k_scale, block_tables[b], L, block_size)
        V = gather_sequence_kv(v_pool, v_scale, block_tables[b], L, block_size)
        pos = np.arange(L)
        for j in range(nq):
            visible = pos <= L - nq + j
            for h in range(Hq):
                s = float(scale) * (K[h // g] @ q[b, j, h].astype(np.float64))
                s = np.where(visible, s, -np.inf)
                w = np.exp(s - np.max(s))
                out[b, j, h] = (w / np.sum(w)) @ V[h // g]
    return out
