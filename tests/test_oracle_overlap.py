"""Pins of the overlap and similarity-pattern oracle (oracle/overlap.py)."""
import json
import os
from itertools import combinations

import numpy as np
import pytest

from oracle import overlap as O
from dsa_inputs import make_correlated_topk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "overlap_tiny.json")


def test_golden_example():
    g = json.load(open(GOLDEN))
    inter = O.overlap_counts(np.array(g["idx"]), g["n_k"])
    assert inter.tolist() == g["inter"]
    for nf, pat in g["patterns"].items():
        assert O.similarity_pattern(inter, int(nf)) == pat
        assert O.similarity_pattern_bruteforce(inter, int(nf)) == pat
        full = [i for i, c in enumerate(pat) if c == "F"]
        assert O.pattern_value(inter, full) == g["values"][nf]


def test_shifted_windows_closed_form():
    """Row r of layer l is the window [s_l + r, s_l + r + k): |A & B| = max(0, k - |s_a - s_b|)."""
    k, R, shifts = 16, 3, [0, 3, 7, 30]
    n_k = 100
    idx = np.array([[np.arange(s + r, s + r + k) for r in range(R)] for s in shifts])
    inter = O.overlap_counts(idx, n_k)
    for a, sa in enumerate(shifts):
        for b, sb in enumerate(shifts):
            assert inter[a, b] == R * max(0, k - abs(sa - sb))


def test_invariants():
    idx = make_correlated_topk(6, 5, 32, 400, swap=0.2, seed=3, short_rows=3)
    inter = O.overlap_counts(idx, 400)
    assert np.array_equal(inter, inter.T)
    valid = (idx >= 0) & (idx < 400)
    assert np.array_equal(np.diag(inter), valid.sum(axis=(1, 2)))
    assert np.all(inter <= np.diag(inter)[:, None]) and np.all(inter >= 0)
    # order of entries inside a row and invalid entries do not matter
    rng = np.random.default_rng(0)
    shuffled = np.array([[rng.permutation(row) for row in layer] for layer in idx])
    assert np.array_equal(O.overlap_counts(shuffled, 400), inter)
    junk = idx.copy()
    junk[junk < 0] = 400 + 7          # out of range instead of -1
    assert np.array_equal(O.overlap_counts(junk, 400), inter)
    # identical layers overlap fully; adjacent layers of the random walk share 1 - swap of a full row
    ratio = O.overlap_ratio(inter)
    assert np.allclose(np.diag(ratio), 1.0)
    full_rows = slice(3, 5)
    sub = O.overlap_counts(idx[:, full_rows], 400)
    assert sub[0, 1] == 2 * (32 - round(0.2 * 32))


@pytest.mark.parametrize("seed", range(12))
def test_dp_equals_bruteforce(seed):
    """The segment recursion finds the brute-force optimum and tie choice,
    on random matrices with many equal totals (small values)."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 10))
    X = rng.integers(0, 4 if seed % 2 else 1000, size=(n, n))
    X = X + X.T
    for nf in range(1, n + 1):
        a = O.similarity_pattern(X, nf)
        b = O.similarity_pattern_bruteforce(X, nf)
        assert a == b, (n, nf)
        full = [i for i, c in enumerate(a) if c == "F"]
        best = max(O.pattern_value(X, (0,) + rest) for rest in combinations(range(1, n), nf - 1))
        assert O.pattern_value(X, full) == best and len(full) == nf and a[0] == "F"


def test_block_structure_gives_block_starts():
    """Layers that reset every 4 layers (blocks of highly similar layers, no
    overlap across blocks): with one F per block the optimum is the uniform
    freq-4 pattern."""
    n, R, k = 12, 4, 64
    idx = make_correlated_topk(n, R, k, 100000, swap=0.05, seed=5, reset_every=4)
    inter = O.overlap_counts(idx, 100000)
    assert O.similarity_pattern(inter, 3) == "FSSS" * 3


def test_reuse_is_from_the_previous_f_layer():
    """S layers reuse the last F layer before them: layer 1 shares much with
    layer 0 and nothing with layer 2, layer 3 a little with layer 2."""
    X = np.array([[9, 8, 0, 0], [8, 9, 0, 0], [0, 0, 9, 1], [0, 0, 1, 9]])
    assert O.similarity_pattern(X, 2) == "FSFS"
    assert O.pattern_value(X, [0, 2]) == 8 + 1
    assert O.pattern_value(X, [0, 3]) == 8 + 0
