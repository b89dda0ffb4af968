"""High-precision brute force for tiny inputs (oracle self-check only).

Written independently of attention.py / append.py: plain Python loops over
Decimal (50 significant digits) and mpmath, with no numpy arithmetic, so a
dropped term, a wrong index or a transposed operand in the float64 oracle
shows up as a disagreement far above float64 rounding.

attn_brute   - softmax(scale * q.K) V per (b, h), walking the block table
               token by token (logical token t lives in physical block
               table[t // BS] at row t % BS).
weights_brute - the softmax weights alone, same walk.
rope_brute   - RMSNorm + split-half RoPE of one head vector at one position.
"""

from decimal import Decimal, getcontext

import mpmath

PREC = 50


def _dec(x) -> Decimal:
    return Decimal(float(x))  # exact: every float is a finite binary fraction


def attn_brute(q, k_vals, v_vals, block_tables, context_lens, scale, block_size=16):
    """Attention over a paged pool given as already-decoded float values.

    q: nested lists / arrays [B][Hq][D]; k_vals, v_vals: [NB][Hkv][BS][D]
    real values (float16 or dequantised E4M3, all exactly representable as
    float64).  Returns a list [B][Hq][D] of Decimal.
    """
    getcontext().prec = PREC
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k_vals[0])
    g = Hq // Hkv
    sc = _dec(scale)
    out = []
    for b in range(B):
        L = int(context_lens[b])
        rows = []
        for h in range(Hq):
            j = h // g
            qh = [_dec(q[b][h][d]) for d in range(D)]
            logits = []
            for t in range(L):
                blk = int(block_tables[b][t // block_size])
                off = t % block_size
                dot = sum((qh[d] * _dec(k_vals[blk][j][off][d]) for d in range(D)),
                          Decimal(0))
                logits.append(sc * dot)
            if L == 0:
                rows.append([Decimal(0)] * D)
                continue
            mx = max(logits)
            w = [(s - mx).exp() for s in logits]
            z = sum(w, Decimal(0))
            o = []
            for d in range(D):
                acc = Decimal(0)
                for t in range(L):
                    blk = int(block_tables[b][t // block_size])
                    acc += w[t] * _dec(v_vals[blk][j][t % block_size][d])
                o.append(acc / z)
            rows.append(o)
        out.append(rows)
    return out


def weights_brute(q, k_vals, block_tables, context_lens, scale, block_size=16):
    """Softmax weights [B][Hq][L_b] as Decimal, token by token."""
    getcontext().prec = PREC
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    g = Hq // len(k_vals[0])
    out = []
    for b in range(B):
        rows = []
        for h in range(Hq):
            s = []
            for t in range(int(context_lens[b])):
                blk = int(block_tables[b][t // block_size])
                s.append(_dec(scale) * sum((_dec(q[b][h][d]) * _dec(k_vals[blk][h // g][t % block_size][d])
                                            for d in range(D)), Decimal(0)))
            mx = max(s) if s else Decimal(0)
            w = [(x - mx).exp() for x in s]
            z = sum(w, Decimal(0))
            rows.append([x / z for x in w])
        out.append(rows)
    return out


def rope_brute(x, gamma, pos, eps, theta):
    """RMSNorm + split-half RoPE of one head vector, mpmath at 50 digits."""
    mpmath.mp.dps = PREC
    D = len(x)
    half = D // 2
    xs = [mpmath.mpf(float(v)) for v in x]
    ms = mpmath.fsum([v * v for v in xs]) / D
    inv = 1 / mpmath.sqrt(ms + mpmath.mpf(float(eps)))
    r = [xs[i] * inv * mpmath.mpf(float(gamma[i])) for i in range(D)]
    y = [None] * D
    th = mpmath.mpf(float(theta))
    for i in range(half):
        a = mpmath.mpf(int(pos)) * mpmath.power(th, mpmath.mpf(-2 * i) / D)
        c, s = mpmath.cos(a), mpmath.sin(a)
        y[i] = r[i] * c - r[i + half] * s
        y[i + half] = r[i + half] * c + r[i] * s
    return y
