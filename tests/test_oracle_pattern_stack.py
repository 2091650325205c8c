"""Pins of the oracle's pattern resolver and layer stack (no GPU)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import PatternError, resolve_pattern
from dsa_inputs import make_indexer_inputs, make_attn_inputs, host_bits, seeded_pattern

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_readme_examples():
    # README, Option A: index_topk_freq=2 makes every 2nd layer Full (half removed)
    p2 = resolve_pattern(47, freq=2)
    assert p2.count("F") == 24 and p2.startswith("FSFS")
    # README, "Which to use?": index_topk_freq 4 keeps a quarter of the indexers
    p4 = resolve_pattern(47, freq=4)
    assert p4.count("F") == 12 and p4.startswith("FSSSFSSSF")
    # README, Default behavior: neither key set -> every layer runs its indexer
    assert resolve_pattern(47) == "F" * 47
    assert resolve_pattern(5, freq=1) == "FFFFF"


def test_glm5_pattern_string():
    g = json.load(open(os.path.join(GOLDEN, "glm5_pattern.json")))
    p = resolve_pattern(g["n_layers"], g["pattern"])
    assert p == g["pattern"]
    assert p.count("F") == g["n_full"] and p.count("S") == g["n_shared"]


@pytest.mark.parametrize("args", [
    (4, "FSF", 0),        # wrong length
    (4, "FSXF", 0),       # bad character
    (4, "fsfs", 0),       # case-sensitive
    (4, "SFFF", 0),       # S before any F
    (4, "FSFS", 2),       # both keys set
    (4, None, -1),        # negative freq
    (0, None, 0),         # no layers
])
def test_pattern_errors(args):
    with pytest.raises(PatternError):
        resolve_pattern(*args)


def test_seeded_pattern():
    p = seeded_pattern(47, 12, seed=9)
    assert len(p) == 47 and p[0] == "F" and p.count("F") == 12
    assert p == seeded_pattern(47, 12, seed=9)


def _layers(n, L=24, H=4, D=16, Ha=2, Da=16, config=96):
    out = []
    for l in range(n):
        ii = make_indexer_inputs(1, L, L, H, D, config=config, layer=l)
        aa = make_attn_inputs(1, L, L, Ha, Da, config=config, layer=l)
        out.append(dict(q_idx=host_bits(ii.q), k_idx=host_bits(ii.k), w=host_bits(ii.w),
                        dtype="bf16", q=host_bits(aa.q), k=host_bits(aa.k), v=host_bits(aa.v)))
    return out


def test_stack_invariants():
    layers = _layers(6)
    k = 5
    P, idx, out, _ = oracle.run_stack(layers, k, pattern="FSSFSF")
    assert P == "FSSFSF"
    # S layers reuse the preceding F layer's indices bitwise (Figure 2 caption)
    assert np.array_equal(idx[1], idx[0]) and np.array_equal(idx[2], idx[0])
    assert np.array_equal(idx[4], idx[3])
    # all-F == running every layer's own indexer; default == freq 1 == 'F'*n
    Pf, idx_f, out_f, _ = oracle.run_stack(layers, k)
    _, idx_1, out_1, _ = oracle.run_stack(layers, k, freq=1)
    assert Pf == "F" * 6
    for l in range(6):
        sc = oracle.indexer_scores_rows(layers[l]["q_idx"], layers[l]["k_idx"], layers[l]["w"],
                                        range(24))
        assert np.array_equal(idx_f[l], oracle.topk_from_scores(sc, k))
        assert np.array_equal(idx_1[l], idx_f[l])
        assert np.array_equal(out_1[l], out_f[l])
    # F layers of any pattern equal the all-F run's same layers
    for l in (0, 3, 5):
        assert np.array_equal(idx[l], idx_f[l])
        assert np.array_equal(out[l], out_f[l])
    # reuse is not equality: an S layer's selection differs from its own indexer's
    assert not np.array_equal(idx[1], idx_f[1])
    assert not np.allclose(out[1], out_f[1])


def test_stack_freq_matches_explicit_pattern():
    layers = _layers(5)
    P, idx, out, _ = oracle.run_stack(layers, 4, freq=2)
    P2, idx2, out2, _ = oracle.run_stack(layers, 4, pattern="FSFSF")
    assert P == P2 == "FSFSF"
    for a, b in zip(idx, idx2):
        assert np.array_equal(a, b)
