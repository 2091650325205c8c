"""GPU parity of dsa_topk_overlap against the oracle (exact integers)."""
import numpy as np
import pytest
import torch

from oracle import overlap as O
from dsa_inputs import make_correlated_topk, make_indexer_inputs
from _gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,R,k,n_k,short", [
    (8, 64, 256, 20000, 10),      # causal short rows padded with -1
    (5, 33, 100, 777, 0),         # layer count not a multiple of the 4-layer rounds; ragged k
    (7, 16, 2048, 1 << 19, 4),    # largest supported n_k
    (1, 3, 16, 50, 3),
])
def test_overlap_random_walk(dsa, n, R, k, n_k, short):
    say(f"overlap n={n} R={R} k={k} n_k={n_k}")
    idx = make_correlated_topk(n, R, k, n_k, swap=0.2, seed=n * 1000 + R, short_rows=short)
    got = dsa.topk_overlap(torch.from_numpy(idx).cuda(), n_k)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.overlap_counts(idx, n_k))


def test_overlap_of_indexer_layers(dsa):
    """Indices from the indexer itself (4 layers, L = 256, k = 16: early rows
    hold -1 padding), and out-of-range junk entries that must be ignored."""
    say("overlap of indexer layers")
    outs = []
    for l in range(4):
        inp = make_indexer_inputs(1, 256, 256, 4, 32, config=1, layer=l).to("cuda")
        outs.append(dsa.indexer_scores_topk(inp.q, inp.k, inp.w, 16).idx[0])
    idx = torch.stack(outs).contiguous()
    idx[2, 100, 3] = 256 + 5          # past n_k: ignored, like -1
    got = dsa.topk_overlap(idx, 256)
    torch.cuda.synchronize()
    ref = O.overlap_counts(idx.cpu().numpy(), 256)
    assert np.array_equal(got.cpu().numpy(), ref)
    again = dsa.topk_overlap(idx, 256)
    torch.cuda.synchronize()
    assert torch.equal(got, again)


def test_overlap_model_size_sampled(dsa):
    """47 layers, 256 query rows, k = 2048 over a 200K context: layer pairs
    sampled against the oracle, every entry checked for symmetry and the
    diagonal against the valid counts, and the similarity pattern from the
    GPU's matrix equals the oracle's pattern from the same matrix."""
    say("overlap 47 layers, k=2048, n_k=200000")
    n, R, k, n_k = 47, 256, 2048, 200000
    idx = make_correlated_topk(n, R, k, n_k, swap=0.1, seed=47, reset_every=6, short_rows=8)
    got = dsa.topk_overlap(torch.from_numpy(idx).cuda(), n_k).cpu().numpy()
    assert np.array_equal(got, got.T)
    assert np.array_equal(np.diag(got), ((idx >= 0) & (idx < n_k)).sum(axis=(1, 2)))
    rng = np.random.default_rng(0)
    for _ in range(6):
        a, b = (int(x) for x in rng.choice(n, 2, replace=False))
        sub = O.overlap_counts(idx[[a, b]], n_k)
        assert sub[0, 1] == got[a, b], (a, b)
    assert dsa.similarity_pattern(got, 12) == O.similarity_pattern(got, 12)
