"""dsa_similarity_pattern (pure host code) against the oracle, and host-side
validation of dsa_topk_overlap. No GPU needed."""
import ctypes
import json
import os

import numpy as np
import pytest

import dsa_indexer_top_amd as dsa
from dsa_indexer_top_amd import _lib as L
from oracle import overlap as O
from dsa_inputs import make_correlated_topk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "overlap_tiny.json")


def test_golden_patterns():
    g = json.load(open(GOLDEN))
    for nf, pat in g["patterns"].items():
        assert dsa.similarity_pattern(np.array(g["inter"]), int(nf)) == pat


@pytest.mark.parametrize("seed", range(16))
def test_pattern_matches_oracle_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 11))
    X = rng.integers(0, 3 if seed % 2 else 10 ** 6, size=(n, n))
    X = X + X.T
    for nf in range(1, n + 1):
        assert dsa.similarity_pattern(X, nf) == O.similarity_pattern_bruteforce(X, nf)


@pytest.mark.parametrize("n,nf", [(47, 12), (78, 40), (61, 16)])
def test_pattern_matches_oracle_at_model_sizes(n, nf):
    """Overlap of a correlated random walk over n layers (the 30B model has 47
    DSA layers, GLM-5 78), n_full as in the pages' 1/4 and 1/2 retention."""
    idx = make_correlated_topk(n, 3, 64, 5000, swap=0.15, seed=n, reset_every=7)
    inter = O.overlap_counts(idx, 5000)
    got = dsa.similarity_pattern(inter, nf)
    assert got == O.similarity_pattern(inter, nf)
    assert got.count("F") == nf and got[0] == "F"
    assert dsa.resolve_pattern(n, got) == got      # a valid stack pattern


def test_pattern_validation(lib=None):
    lib = dsa.load()
    X = (ctypes.c_int64 * 4)(1, 0, 0, 1)
    out = ctypes.create_string_buffer(3)
    assert lib.dsa_similarity_pattern(2, X, 0, out) == L.DSA_ERR_INVALID_ARGUMENT
    assert lib.dsa_similarity_pattern(2, X, 3, out) == L.DSA_ERR_INVALID_ARGUMENT
    assert lib.dsa_similarity_pattern(0, X, 1, out) == L.DSA_ERR_INVALID_ARGUMENT
    assert lib.dsa_similarity_pattern(2, None, 1, out) == L.DSA_ERR_INVALID_ARGUMENT
    neg = (ctypes.c_int64 * 4)(1, -1, 0, 1)
    assert lib.dsa_similarity_pattern(2, neg, 1, out) == L.DSA_ERR_INVALID_ARGUMENT
    assert lib.dsa_similarity_pattern(2, X, 2, out) == L.DSA_OK and out.value == b"FF"


def test_overlap_validation():
    lib = dsa.load()
    FAKE = 1 << 20
    f = lib.dsa_topk_overlap
    assert f(FAKE, 0, 4, 16, 100, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 1025, 4, 16, 100, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 4, 0, 16, 100, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 4, 4, 0, 100, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 4, 4, 16, (1 << 19) + 1, FAKE, None) == L.DSA_ERR_UNSUPPORTED
    assert f(FAKE, 4, 4, 16, 0, FAKE, None) == L.DSA_ERR_UNSUPPORTED
    assert f(None, 4, 4, 16, 100, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 4, 4, 16, 100, FAKE + 4, None) == L.DSA_ERR_INVALID_ARGUMENT   # inter not 8-byte aligned
