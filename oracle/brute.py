"""Pure-Python brute-force references for tiny inputs (test infrastructure).

Written independently of the NumPy oracle: every sum is an explicit loop, the
top-k is a full sort of all candidates, and attention is computed with
math.exp. Used only to pin the NumPy oracle on tiny shapes. Values are taken as
Python floats (or exact fractions when the inputs are given as Fractions).
"""
from __future__ import annotations

import math


def brute_scores(Q, K, W, pos_offset=0):
    """Q: nested lists [n_q][H][D]; K: [n_k][D]; W: [n_q][H]. Returns a dict
    {(t, s): score} over causal pairs s <= pos_offset + t, s < n_k."""
    out = {}
    n_k = len(K)
    for t in range(len(Q)):
        p = pos_offset + t
        for s in range(n_k):
            if s > p:
                continue
            total = 0
            for j in range(len(Q[t])):
                dot = 0
                for c in range(len(K[s])):
                    dot += Q[t][j][c] * K[s][c]
                if dot > 0:
                    total += W[t][j] * dot
            out[(t, s)] = total
    return out


def brute_topk(scores, n_q, n_k, k, pos_offset=0):
    """Full sort of each row by (score descending, index ascending)."""
    rows = []
    for t in range(n_q):
        p = pos_offset + t
        cands = [(scores[(t, s)], s) for s in range(n_k) if s <= p]
        cands.sort(key=lambda x: (-x[0], x[1]))
        chosen = [s for _, s in cands[:k]]
        rows.append(chosen + [-1] * (k - len(chosen)))
    return rows


def brute_attention(q, K, V, sel, scale):
    """One query head: q [D], K/V [n_k][D], sel list of row indices."""
    if not sel:
        return [0.0] * len(V[0]), -math.inf
    a = []
    for s in sel:
        dot = 0.0
        for c in range(len(q)):
            dot += q[c] * K[s][c]
        a.append(scale * dot)
    m = max(a)
    e = [math.exp(x - m) for x in a]
    z = sum(e)
    out = []
    for c in range(len(V[0])):
        acc = 0.0
        for i, s in enumerate(sel):
            acc += e[i] * V[s][c]
        out.append(acc / z)
    return out, m + math.log(z)
