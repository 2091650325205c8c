"""The no-allocation indexer entry point (dsa_indexer_scores_topk_static):
its results equal dsa_indexer_scores_topk's bit for bit, on consecutive calls
whose second input is smaller than the first (the static scratch keeps the
previous call's contents), and a shape beyond the scratch is rejected."""
import pytest
import torch

from dsa_inputs import make_indexer_inputs, make_int_indexer_inputs
from _gpu_helpers import say

pytestmark = pytest.mark.gpu


def _both(dsa, inp, topk):
    g = inp
    kw = dict(q_scale=g.q_scale, k_scale=g.k_scale, pos_offset=g.pos_offset, out_scores=True)
    ref = dsa.indexer_scores_topk(g.q, g.k, g.w, topk, **kw)
    out_idx = torch.full_like(ref.idx, 7)
    out_sc = torch.full_like(ref.scores, 3.0)
    st = dsa.indexer_scores_topk(g.q, g.k, g.w, topk, out_idx=out_idx, static_scratch=True,
                                 **{**kw, "out_scores": out_sc})
    torch.cuda.synchronize()
    assert torch.equal(st.idx, ref.idx), "indices differ from the workspace entry point"
    assert torch.equal(st.scores.view(torch.int32), ref.scores.view(torch.int32)), "scores differ"
    return ref


@pytest.mark.parametrize("case", ["decode", "prefill"])
def test_static_matches_workspace_entry_point(dsa, case):
    """Two calls in a row through the static scratch, the second smaller."""
    if case == "decode":
        shapes = [(32, 1, 200000, "bf16"), (3, 1, 70001, "fp8")]
    else:
        shapes = [(2, 400, 6000, "fp8"), (1, 97, 3001, "bf16")]
    for i, (B, n_q, n_k, dt) in enumerate(shapes):
        say(f"static scratch {case} call {i}: B={B} n_q={n_q} n_k={n_k} {dt}")
        inp = make_indexer_inputs(B, n_q, n_k, 64, 128, config=40 + i, dtype=dt, w_std=0.125, device="cuda")
        _both(dsa, inp, 2048)


def test_static_exact_ties_after_large_call(dsa):
    """Exact-integer inputs (many tied scores: the tie paths read the most
    scratch) right after a large call."""
    say("static scratch ties")
    big = make_indexer_inputs(32, 1, 200000, 64, 128, config=44, w_std=0.125, device="cuda")
    _both(dsa, big, 2048)
    small = make_int_indexer_inputs(2, 1, 3000, 64, 128, seed=13).to("cuda")
    _both(dsa, small, 2048)
    pre = make_int_indexer_inputs(1, 64, 900, 16, 64, seed=14).to("cuda")
    _both(dsa, pre, 100)


def test_static_rejects_oversized_shape(dsa):
    from dsa_indexer_top_amd import _lib as L
    inp = make_indexer_inputs(1, 2000, 2000, 64, 128, config=45, w_std=0.125, device="cuda")
    need = dsa.indexer_workspace_size(1, 2000, 2000, 64, 128, 2048)
    assert need > L.DSA_STATIC_SCRATCH_BYTES
    with pytest.raises(dsa.DsaError) as ei:
        dsa.indexer_scores_topk(inp.q, inp.k, inp.w, 2048, static_scratch=True)
    assert ei.value.status == L.DSA_ERR_WORKSPACE
