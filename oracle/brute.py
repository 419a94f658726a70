"""Scalar pure-Python restatement of the layer for tiny inputs.

Test infrastructure only.  It shares no helper with oracle.csa: rotations are
complex multiplications, softmaxes are explicit sums over Python floats, and
every loop runs over single scalars.  Agreement between the two on tiny inputs
pins the vectorised oracle against slicing, axis and broadcasting mistakes.
Sources as in oracle.csa ([W1] .. [W5]).
"""
from __future__ import annotations

import cmath
import math


def pool_entry(i, m, rows_a, gates_a, bias_a, rows_b=None, gates_b=None, bias_b=None):
    """One entry, channel by channel (W2 compression equation).

    rows_*[r][c] / gates_*[r][c] are the m tokens of the a (current) and b
    (previous) blocks; the b block is omitted for i == 0 or without overlap.
    """
    D = len(rows_a[0])
    out = []
    for c in range(D):
        cand = []
        for r in range(m):
            cand.append((gates_a[r][c] + bias_a[r][c], rows_a[r][c]))
        if rows_b is not None and i >= 1:
            for r in range(m):
                cand.append((gates_b[r][c] + bias_b[r][c], rows_b[r][c]))
        big = max(lg for lg, _ in cand)
        num = 0.0
        den = 0.0
        for lg, v in cand:
            e = math.exp(lg - big)
            num += e * v
            den += e
        out.append(num / den)
    return out


def rms(x, eps=1e-6):
    ss = 0.0
    for v in x:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(x) + eps)
    return [v * r for v in x]


def rotate(x, pos, theta, d_r):
    """Partial RoPE as complex multiplication of the pair (x[2u] + i x[2u+1])
    by exp(i * pos * theta**(-2u/d_r)) in the last d_r dims."""
    d = len(x)
    out = list(x)
    base = d - d_r
    for u in range(d_r // 2):
        z = complex(x[base + 2 * u], x[base + 2 * u + 1])
        z *= cmath.exp(1j * pos * theta ** (-2.0 * u / d_r))
        out[base + 2 * u] = z.real
        out[base + 2 * u + 1] = z.imag
    return out


def index_score(q_heads, w, key):
    tot = 0.0
    for h, qh in enumerate(q_heads):
        dot = 0.0
        for a, b in zip(qh, key):
            dot += a * b
        if dot > 0.0:
            tot += w[h] * dot
    return tot


def select(scores, k):
    """k best by (score desc, index asc), returned ascending and padded with -1."""
    n = len(scores)
    chosen = []
    taken = [False] * n
    for _ in range(min(k, n)):
        best = -1
        for i in range(n):
            if taken[i]:
                continue
            if best < 0 or scores[i] > scores[best]:
                best = i
        taken[best] = True
        chosen.append(best)
    chosen.sort()
    return chosen + [-1] * (k - len(chosen))


def attend(q_heads, t, kv_rows, sink, theta, d_r, scale, norm_q=True, inv_rope=True):
    """One query, every head separately: sink joins the softmax denominator."""
    outs = []
    lses = []
    for h, qh in enumerate(q_heads):
        qv = rms(qh) if norm_q else list(qh)
        qv = rotate(qv, t, theta, d_r)
        s = []
        for row in kv_rows:
            dot = 0.0
            for a, b in zip(qv, row):
                dot += a * b
            s.append(dot * scale)
        big = max(s + [sink[h]])
        den = math.exp(sink[h] - big)
        acc = [0.0] * len(qh)
        tot = 0.0
        for sj, row in zip(s, kv_rows):
            e = math.exp(sj - big)
            den += e
            tot += e
            for c in range(len(acc)):
                acc[c] += e * row[c]
        o = [a / den for a in acc]
        if inv_rope:
            o = rotate(o, -t, theta, d_r)
        outs.append(o)
        lses.append(big + math.log(tot) if tot > 0 else -math.inf)
    return outs, lses
