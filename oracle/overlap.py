"""Cross-layer top-k overlap and a similarity-based F/S pattern, exact integers.

Sources. The IndexCache paper's appendix (Figure 4) plots the pairwise top-k
index overlap ratio between all layer pairs of a DSA model, and Table 5
evaluates a training-free pattern searched from that similarity; the
repository page ("Key Insight") reports that adjacent layers share most of
their selected tokens. The pages give neither the exact ratio nor the search,
so the plain readings below are taken.

Overlap. For index tensors idx[l] of shape [R, k] (the same R query rows for
every layer l), S_l(r) is the set of valid entries (0 <= v < n_k) of row r.
    inter[a][b] = sum_r |S_a(r) & S_b(r)|,    inter[a][a] = sum_r |S_a(r)|,
and the overlap ratio of a and b is inter[a][b] / inter[a][a] (for the
indexer's rows all layers have the same counts, so this is the mean of
|A & B| / k weighted by the rows' sizes).

Similarity-based pattern. With n_full F layers, layer 0 among them, every S
layer l reuses the indices of the last F layer f(l) < l (the IndexCache
buffer rule). The pattern maximises the shared selections
    sum over S layers l of inter[f(l)][l]
over all such patterns; among equal totals, the one whose sorted list of F
layers is lexicographically smallest wins. The exact maximum is taken (by
brute force here for small stacks, and by a segment recursion for any size),
not a greedy approximation.
"""
from __future__ import annotations

from itertools import combinations
from typing import List, Sequence

import numpy as np


def overlap_counts(idx, n_k: int) -> np.ndarray:
    """idx: [n_layers, R, k] integers. Returns inter [n_layers, n_layers] int64."""
    I = np.asarray(idx)
    n, R, _ = I.shape
    sets = [[set(int(v) for v in I[l, r] if 0 <= int(v) < n_k) for r in range(R)] for l in range(n)]
    out = np.zeros((n, n), dtype=np.int64)
    for a in range(n):
        for b in range(n):
            out[a, b] = sum(len(sets[a][r] & sets[b][r]) for r in range(R))
    return out


def overlap_ratio(inter) -> np.ndarray:
    """inter[a][b] / inter[a][a] (0 where a layer selected nothing)."""
    X = np.asarray(inter, dtype=np.float64)
    d = np.diag(X).copy()
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(d[:, None] > 0, X / np.where(d[:, None] > 0, d[:, None], 1.0), 0.0)


def pattern_value(inter, full: Sequence[int]) -> int:
    """Shared selections of the pattern whose F layers are `full`."""
    X = np.asarray(inter)
    n = X.shape[0]
    fs = set(full)
    total, last = 0, None
    for l in range(n):
        if l in fs:
            last = l
        else:
            total += int(X[last, l])
    return total


def _as_pattern(n: int, full: Sequence[int]) -> str:
    fs = set(full)
    return "".join("F" if l in fs else "S" for l in range(n))


def similarity_pattern_bruteforce(inter, n_full: int) -> str:
    """Every choice of the n_full - 1 F layers after layer 0, in lexicographic
    order; the first with the largest total wins (small stacks only)."""
    n = np.asarray(inter).shape[0]
    best, arg = None, None
    for rest in combinations(range(1, n), n_full - 1):
        full = (0,) + rest
        v = pattern_value(inter, full)
        if best is None or v > best:
            best, arg = v, full
    return _as_pattern(n, arg)


def similarity_pattern(inter, n_full: int) -> str:
    """The same optimum for any size. V[i][j]: the best total of layers i..n-1
    when layer i is F and j F layers lie in i..n-1; a segment from F layer i
    to the next F layer e (or the end) contributes sum_{i < l < e} inter[i][l].
    The F layers are then read off front to back, each time the smallest next
    F layer that keeps the optimum."""
    X = np.asarray(inter).astype(object)  # exact integers
    n = X.shape[0]
    if not 1 <= n_full <= n:
        raise ValueError("n_full out of range")

    def seg(i, e):
        return sum(X[i, l] for l in range(i + 1, e))

    NEG = None
    V = [[NEG] * (n_full + 1) for _ in range(n + 1)]
    for i in range(n - 1, -1, -1):
        V[i][1] = seg(i, n)
        for j in range(2, n_full + 1):
            best = NEG
            for e in range(i + 1, n - j + 2):
                if V[e][j - 1] is None:
                    continue
                v = seg(i, e) + V[e][j - 1]
                if best is None or v > best:
                    best = v
            V[i][j] = best
    full: List[int] = [0]
    i, j = 0, n_full
    while j > 1:
        target = V[i][j]
        for e in range(i + 1, n - j + 2):
            if V[e][j - 1] is not None and seg(i, e) + V[e][j - 1] == target:
                full.append(e)
                i, j = e, j - 1
                break
    return _as_pattern(n, full)
