"""GPU parity of chunked prefill through the layer stack
(dsa_layer_stack_run_chunked): one sequence prefilled in chunks of query rows
over the keys cached so far must give the one-shot stack's results."""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import host_bits, make_attn_inputs, make_indexer_inputs
from _gpu_helpers import ATTN_ATOL, say

pytestmark = pytest.mark.gpu


def _layers(n, n_q, n_k, dtype, config):
    out = []
    for l in range(n):
        ii = make_indexer_inputs(1, n_q, n_k, 64, 128, config=config, layer=l, dtype=dtype, w_std=0.125,
                                 device="cuda")
        aa = make_attn_inputs(1, n_q, n_k, 16, 128, config=config, layer=l, device="cuda")
        out.append(dict(q_idx=ii.q, k_idx=ii.k, w=ii.w, q_scale=ii.q_scale, k_scale=ii.k_scale,
                        q=aa.q, k=aa.k, v=aa.v))
    return out


def _run(dsa, layers, topk, pattern, chunk_rows=None, pos_offset=None):
    st = dsa.LayerStack(layers, topk, chunk_rows=chunk_rows, pos_offset=pos_offset, lse=True)
    st.run(pattern)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_chunked_equals_one_shot(dsa, dtype):
    """4 layers 'FSSF' at L = 9000 (H_I = 64, d_I = 128, k = 2048; attention 16
    heads, d = 128) in three ragged chunks of more than 1024 rows: indices and
    every layer's output and lse equal the one-shot run bit for bit."""
    L, topk, pat = 9000, 2048, "FSSF"
    say(f"chunked {dtype}")
    layers = _layers(4, L, L, dtype, config=7)
    one = _run(dsa, layers, topk, pat)
    ch = _run(dsa, layers, topk, pat, chunk_rows=3001)   # 3001, 3001, 2998 rows
    assert ch.idx_buf.shape == (1, 3001, topk)
    assert torch.equal(ch.idx_buf[0, :2998], one.idx_buf[0, 6002:]), "last chunk's indices differ"
    for l in range(4):
        assert torch.equal(ch.outs[l], one.outs[l]), f"layer {l} output differs"
        assert torch.equal(ch.lses[l], one.lses[l]), f"layer {l} lse differs"


def test_chunked_small_chunks_and_decode_tail(dsa):
    """Chunks of 700 rows (attention splits each row in two, unlike the one-shot
    run) and a one-row last chunk (the decode kernels): every layer's outputs
    within the attention tolerance of the oracle over the one-shot run's
    indices, and the tail row selects the one-shot row's tokens up to
    near-ties."""
    L, topk, pat = 4201, 2048, "FSF"
    say("chunked small")
    layers = _layers(3, L, L, "bf16", config=8)
    one = _run(dsa, layers, topk, pat)
    ch = _run(dsa, layers, topk, pat, chunk_rows=700)    # 6 x 700 + 1 row
    # the one-row tail runs the decode kernels: same selection up to near-ties
    tail = set(ch.idx_buf[0, 0].tolist())
    ref_tail = set(one.idx_buf[0, L - 1].tolist())
    assert -1 not in tail and len(tail & ref_tail) >= 0.99 * topk
    rows = [0, 699, 700, 2047, 2048, 4199]
    # the F layers' own selections: layer 0 (used by layers 0 and 1) and layer 2
    idx0 = dsa.indexer_scores_topk(layers[0]["q_idx"], layers[0]["k_idx"], layers[0]["w"], topk).idx
    torch.cuda.synchronize()
    sel = {0: idx0[0].cpu().numpy(), 1: idx0[0].cpu().numpy(), 2: one.idx_buf[0].cpu().numpy()}
    for l in range(3):
        gi = sel[l]
        a = layers[l]
        ka, va = host_bits(a["k"]), host_bits(a["v"])
        ref = np.stack([oracle.sparse_attention_rows(host_bits(a["q"][:, [t]]), ka, va, gi[[t]], [0],
                                                     pos_offset=t)[0][0] for t in rows])
        got = ch.outs[l][0, rows].float().cpu().numpy()
        err = np.abs(got - ref).max()
        assert err <= ATTN_ATOL, f"layer {l}: {err}"
        # rows of the 700-row chunks: same indices, a different split of the row
        assert (ch.outs[l][0, :L - 1].float() - one.outs[l][0, :L - 1].float()).abs().max().item() <= ATTN_ATOL


def test_chunked_over_cached_prefix(dsa):
    """Queries at positions 3000..8999 over 9000 keys (a cached prefix of 3000
    tokens), chunks of 2500 rows: equal to the one-shot run with the same
    offset, bit for bit."""
    n_k, n_q, topk, pat = 9000, 6000, 2048, "FS"
    say("chunked prefix")
    layers = _layers(2, n_q, n_k, "fp8", config=9)
    one = _run(dsa, layers, topk, pat, pos_offset=n_k - n_q)
    ch = _run(dsa, layers, topk, pat, chunk_rows=2500, pos_offset=n_k - n_q)   # 2500, 2500, 1000
    assert torch.equal(ch.idx_buf[0, :1000], one.idx_buf[0, 5000:])
    # chunks 0 and 1 have more than 1024 rows: bit for bit; the 1000-row chunk splits rows in two
    for l in range(2):
        assert torch.equal(ch.outs[l][0, :5000], one.outs[l][0, :5000])
        assert (ch.outs[l][0, 5000:].float() - one.outs[l][0, 5000:].float()).abs().max().item() <= ATTN_ATOL
