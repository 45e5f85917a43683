"""Loop-by-loop restatement of the path for tiny inputs (pure Python floats).

It is written differently from ``method`` on purpose — dense masks over every
key instead of gathered key lists, Python ``sorted`` instead of NumPy sorting,
scalar ``math.exp`` instead of vector softmax — so that agreement between the
two pins both against slips in indexing, masking and tie handling.
"""
from __future__ import annotations

import math


def compress(x, gate, pos_bias, m):
    B, T, C = len(x), len(x[0]), len(x[0][0])
    out = []
    for b in range(B):
        yb = []
        for i in range(T // m):
            z = [gate[b][i * m + j] + pos_bias[j] for j in range(m)]
            zmax = max(z)
            e = [math.exp(v - zmax) for v in z]
            tot = sum(e)
            yb.append([sum(e[j] / tot * x[b][i * m + j][c] for j in range(m)) for c in range(C)])
        out.append(yb)
    return out


def score(qh, w, kj):
    """sum over indexer heads of w_h * relu(q_h . k_j)."""
    tot = 0.0
    for h in range(len(qh)):
        d = sum(qh[h][t] * kj[t] for t in range(len(kj)))
        tot += w[h] * (d if d > 0 else 0.0)
    return tot


def select(scores, n, k):
    """k best of the first n scores, larger first, ties to the lower index; ascending."""
    best = sorted(range(n), key=lambda j: (-scores[j], j))[: min(k, n)]
    return sorted(best) + [-1] * (k - min(k, n))


def attend_masked(q, kc, vc, chosen, kw, vw, win_pos0, W, p, scale):
    """One query, one head: masked softmax over ALL compressed rows and ALL window rows."""
    logits, vals = [], []
    for j in range(len(kc)):
        if j in chosen:
            logits.append(scale * sum(q[d] * kc[j][d] for d in range(len(q))))
            vals.append(vc[j])
    for r in range(len(kw)):
        pos = win_pos0 + r
        if p - W < pos <= p:
            logits.append(scale * sum(q[d] * kw[r][d] for d in range(len(q))))
            vals.append(vw[r])
    if not logits:
        return [0.0] * len(q), -math.inf
    zmax = max(logits)
    e = [math.exp(z - zmax) for z in logits]
    tot = sum(e)
    o = [sum(e[i] * vals[i][d] for i in range(len(e))) / tot for d in range(len(vc[0]) if vc else len(q))]
    return o, zmax + math.log(tot)
