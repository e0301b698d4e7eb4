"""Pure-Python brute force of the self-attention block, for tiny inputs only.

Written straight from the definition with lists, loops, ``math.exp`` and
``math.fsum``, independently of the numpy oracle (it shares no code with it).
Block definition: "Tensor Parallelism: Sharding Weights for Parallel Layer
Execution", section 3 (project, split heads, scaled dot-product attention,
concatenate and project with W_O); Y = X A with A [h_in, h_out] (section 1).

Here the 1/sqrt(d) factor multiplies each dot product, not the query, so the
two implementations also round differently.
"""

from __future__ import annotations

import math


def _tolist(a):
    return [[float(v) for v in row] for row in a]


def matmul(a, b):
    n, kk, m = len(a), len(b), len(b[0])
    assert len(a[0]) == kk
    return [[math.fsum(a[i][t] * b[t][j] for t in range(kk)) for j in range(m)] for i in range(n)]


def block(x, wq, wk, wv, wo, num_heads):
    """Return (y [S][h], o [S][h], lse [H][S]) as nested lists."""
    x, wq, wk, wv, wo = (_tolist(a) for a in (x, wq, wk, wv, wo))
    s, h = len(x), len(x[0])
    d = h // num_heads
    q = matmul(x, wq)
    k = matmul(x, wk)
    v = matmul(x, wv)
    scale = 1.0 / math.sqrt(d)
    o = [[0.0] * h for _ in range(s)]
    lse = [[0.0] * s for _ in range(num_heads)]
    for j in range(num_heads):
        cols = range(j * d, (j + 1) * d)
        for i in range(s):
            scores = [scale * math.fsum(q[i][c] * k[t][c] for c in cols) for t in range(s)]
            m = max(scores)
            e = [math.exp(sc - m) for sc in scores]
            z = math.fsum(e)
            for c in cols:
                o[i][c] = math.fsum(e[t] * v[t][c] for t in range(s)) / z
            lse[j][i] = m + math.log(z)
    y = matmul(o, wo)
    return y, o, lse


def attention_one_head(q_scaled, k, v):
    """Brute-force attention of one head with an already scaled query."""
    q_scaled, k, v = (_tolist(a) for a in (q_scaled, k, v))
    out, lses = [], []
    for qi in q_scaled:
        scores = [math.fsum(a * b for a, b in zip(qi, kt)) for kt in k]
        m = max(scores)
        e = [math.exp(sc - m) for sc in scores]
        z = math.fsum(e)
        out.append([math.fsum(e[t] * k_v for t, k_v in enumerate(col)) / z
                    for col in zip(*v)])
        lses.append(m + math.log(z))
    return out, lses


def rms_norm(x, gain, eps):
    """Brute-force RMSNorm of each row: x_j / sqrt(mean of squares + eps) * g_j."""
    out = []
    for row in _tolist(x):
        ms = math.fsum(v * v for v in row) / len(row)
        inv = 1.0 / math.sqrt(ms + eps)
        out.append([v * inv * (1.0 if gain is None else float(gain[j])) for j, v in enumerate(row)])
    return out


def ulysses_recv_blocks(t, n_ranks, rank, keys_last=False):
    """Brute-force first all-to-all on nested lists: t [H][S][d] (or [H][d][S]
    with keys_last); returns block p for every p as nested lists."""
    hh = len(t)
    hl = hh // n_ranks
    heads = range(rank * hl, (rank + 1) * hl)
    out = []
    for p in range(n_ranks):
        blk = []
        for j in heads:
            if keys_last:
                s = len(t[j][0])
                c = s // n_ranks
                blk.append([[t[j][dd][p * c + i] for i in range(c)] for dd in range(len(t[j]))])
            else:
                s = len(t[j])
                c = s // n_ranks
                blk.append([list(t[j][p * c + i]) for i in range(c)])
        out.append(blk)
    return out


def tp_share(x, wq, wk, wv, wo, num_heads, n_ranks, rank):
    """Brute-force TP partial output of one rank (nested lists)."""
    x, wq, wk, wv, wo = (_tolist(a) for a in (x, wq, wk, wv, wo))
    s, h = len(x), len(x[0])
    d = h // num_heads
    hl = num_heads // n_ranks
    cols = list(range(rank * hl * d, (rank + 1) * hl * d))
    sub = lambda w: [[w[i][c] for c in cols] for i in range(h)]
    q, k, v = matmul(x, sub(wq)), matmul(x, sub(wk)), matmul(x, sub(wv))
    scale = 1.0 / math.sqrt(d)
    o = [[0.0] * len(cols) for _ in range(s)]
    for j in range(hl):
        cc = range(j * d, (j + 1) * d)
        for i in range(s):
            sc = [scale * math.fsum(q[i][c] * k[t][c] for c in cc) for t in range(s)]
            m = max(sc)
            e = [math.exp(a - m) for a in sc]
            z = math.fsum(e)
            for c in cc:
                o[i][c] = math.fsum(e[t] * v[t][c] for t in range(s)) / z
    wo_rows = [wo[c] for c in cols]
    return matmul(o, wo_rows)
