"""GPU parity of dsa_sparse_attn and dsa_layer_stack_run against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import (host_bits, make_attn_inputs, make_indexer_inputs, seeded_pattern)
from _gpu_helpers import ATTN_ATOL, overlap, say

pytestmark = pytest.mark.gpu


def _random_idx(B, n_q, n_k, topk, off, seed, junk=False):
    rng = np.random.default_rng(seed)
    idx = np.full((B, n_q, topk), -1, np.int32)
    for b in range(B):
        for t in range(n_q):
            p = off + t
            n = min(topk, p + 1)
            idx[b, t, :n] = rng.choice(p + 1, n, replace=False)
            if junk and topk > n + 1:
                idx[b, t, n] = p + 1 + rng.integers(0, 5)   # non-causal entry: skipped
    return idx


def _check_attn(dsa, a, idx, scale=0.0):
    g = a.to("cuda")
    gi = torch.from_numpy(idx).cuda()
    out, lse = dsa.sparse_attn(g.q, g.k, g.v, gi, scale=scale, pos_offset=a.pos_offset, lse=True)
    torch.cuda.synchronize()
    O = out.float().cpu().numpy()
    LS = lse.cpu().numpy()
    ref_o, ref_l = oracle.sparse_attention(host_bits(a.q), host_bits(a.k), host_bits(a.v), idx,
                                           scale=scale or None, pos_offset=a.pos_offset)
    err = np.abs(O - ref_o).max()
    assert err <= ATTN_ATOL, f"attention max-abs error {err}"
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(LS))
    assert np.abs(LS[fin] - ref_l[fin]).max() <= 1e-3 * (1 + np.abs(ref_l[fin]).max())
    return O, LS, err


@pytest.mark.parametrize("B,L,H,D,topk,junk", [
    (1, 256, 4, 64, 16, False),     # tiny stack layer shape
    (1, 300, 16, 128, 64, True),    # ragged chunks, skipped entries
    (2, 70, 16, 64, 40, True),      # D = 64 path, B = 2
    (1, 40, 3, 128, 200, False),    # topk > L: trailing -1
])
def test_attn_random(dsa, B, L, H, D, topk, junk):
    say(f"attn B={B} L={L} H={H} D={D} k={topk}")
    a = make_attn_inputs(B, L, L, H, D, config=30)
    _check_attn(dsa, a, _random_idx(B, L, L, topk, 0, 1, junk))


def test_attn_full_selection_is_dense(dsa):
    """Every causal key selected: the result is dense causal attention."""
    L, H, D = 96, 16, 128
    a = make_attn_inputs(1, L, L, H, D, config=31)
    idx = np.full((1, L, L), -1, np.int32)
    for t in range(L):
        idx[0, t, :t + 1] = np.arange(t + 1)[::-1]
    _check_attn(dsa, a, idx, scale=0.09)


def test_attn_empty_row(dsa):
    L = 8
    a = make_attn_inputs(1, L, L, 4, 64, config=32)
    idx = np.full((1, L, 4), -1, np.int32)
    idx[0, 5, 0] = 2
    O, LS, _ = _check_attn(dsa, a, idx)
    assert np.all(O[0, 0] == 0) and np.all(LS[0, 0] == -np.inf)


@pytest.mark.parametrize("B,n_k,topk", [(3, 5000, 2048), (1, 300, 100), (2, 64, 2048)])
def test_attn_decode_split(dsa, B, n_k, topk):
    say(f"attn decode B={B} n_k={n_k} k={topk}")
    a = make_attn_inputs(B, 1, n_k, 16, 128, config=33)
    _check_attn(dsa, a, _random_idx(B, 1, n_k, topk, n_k - 1, 2))


@pytest.mark.parametrize("B,n_q,n_k,H,D,topk", [
    (1, 2048, 2048, 4, 64, 64),       # one wave per row, two chunks
    (1, 256, 2000, 16, 128, 512),     # 8 splits: one 8-wave workgroup per row merges in LDS
    (1, 128, 3000, 12, 64, 700),      # 16 splits: four 4-wave workgroup partials, ragged last chunk
    (4, 16, 5000, 16, 128, 1500),     # 32 splits: eight 4-wave workgroup partials, empty last splits
    (1, 1, 5000, 5, 64, 2048),        # 64 splits (16 partials), D = 64, 5 heads
    (1, 1024, 3000, 16, 64, 1024),    # 2 splits of 16 chunks each (K of the next chunk read ahead), D = 64
    (1, 2048, 4096, 8, 128, 512),     # one wave per row, 16 chunks (read ahead), D = 128
])
def test_attn_split_forms(dsa, B, n_q, n_k, H, D, topk):
    """Each launch form of the split-K rule (about 2048 waves per call): direct,
    per-wave partials, one 8-wave workgroup per row merging in LDS, and 4-wave
    workgroups writing 4..16 partials; with one chunk per wave and with several
    (the next chunk's K read ahead)."""
    say(f"attn forms B={B} n_q={n_q} n_k={n_k} H={H} D={D} k={topk}")
    a = make_attn_inputs(B, n_q, n_k, H, D, config=34)
    _check_attn(dsa, a, _random_idx(B, n_q, n_k, topk, n_k - n_q, 3, junk=True))


# ------------------------------------------------------------------ stack
def _stack_layers(n_layers, L, H_I, D_I, H, D, config, dtype="bf16"):
    dev, host = [], []
    for l in range(n_layers):
        ii = make_indexer_inputs(1, L, L, H_I, D_I, config=config, layer=l, dtype=dtype)
        aa = make_attn_inputs(1, L, L, H, D, config=config, layer=l)
        g, ga = ii.to("cuda"), aa.to("cuda")
        dev.append(dict(q_idx=g.q, k_idx=g.k, w=g.w, q_scale=g.q_scale, k_scale=g.k_scale,
                        q=ga.q, k=ga.k, v=ga.v))
        host.append(dict(q_idx=host_bits(ii.q), k_idx=host_bits(ii.k), w=host_bits(ii.w),
                         q_scale=host_bits(ii.q_scale), k_scale=host_bits(ii.k_scale), dtype=dtype,
                         q=host_bits(aa.q), k=host_bits(aa.k), v=host_bits(aa.v)))
    return dev, host


def test_stack_tiny_fsfs(dsa):
    """The tiny 4-layer 'FSFS' stack: S layers reuse the preceding F layer's
    indices, every layer matches separate indexer/attention calls bitwise, and
    the result matches the oracle stack."""
    say("stack FSFS")
    L, k = 256, 16
    dev, host = _stack_layers(4, L, 4, 32, 4, 64, config=1)
    st = dsa.LayerStack(dev, k, lse=True)
    st.run("FSFS")
    torch.cuda.synchronize()
    outs = [o.clone() for o in st.outs]
    # separate calls
    idx0 = dsa.indexer_scores_topk(dev[0]["q_idx"], dev[0]["k_idx"], dev[0]["w"], k).idx
    idx2 = dsa.indexer_scores_topk(dev[2]["q_idx"], dev[2]["k_idx"], dev[2]["w"], k).idx
    assert torch.equal(st.idx_buf, idx2)
    for l, ix in ((0, idx0), (1, idx0), (2, idx2), (3, idx2)):
        o, _ = dsa.sparse_attn(dev[l]["q"], dev[l]["k"], dev[l]["v"], ix)
        assert torch.equal(o, outs[l]), f"layer {l} differs from a separate call"
    torch.cuda.synchronize()
    # oracle stack
    P, ridx, _, _ = oracle.run_stack(host, k, pattern="FSFS")
    assert P == "FSFS"
    for l, ix in ((0, idx0), (2, idx2)):
        ov, _ = overlap(ix.cpu().numpy()[0], ridx[l])
        assert ov >= 0.99
        ref, _ = oracle.sparse_attention_rows(host[l]["q"], host[l]["k"], host[l]["v"],
                                              ix.cpu().numpy()[0], range(L))
        assert np.abs(outs[l].float().cpu().numpy()[0] - ref).max() <= ATTN_ATOL
    ref3, _ = oracle.sparse_attention_rows(host[3]["q"], host[3]["k"], host[3]["v"],
                                           idx2.cpu().numpy()[0], range(L))
    assert np.abs(outs[3].float().cpu().numpy()[0] - ref3).max() <= ATTN_ATOL
    # reuse is not equality: layer 1 with its own indexer would select differently
    own1 = dsa.indexer_scores_topk(dev[1]["q_idx"], dev[1]["k_idx"], dev[1]["w"], k).idx
    assert not torch.equal(own1, idx0)


def test_stack_patterns_and_determinism(dsa):
    say("stack patterns")
    L, k, n = 200, 32, 6
    dev, _ = _stack_layers(n, L, 64, 128, 16, 128, config=3)
    st = dsa.LayerStack(dev, k)

    def run(pattern=None, freq=0):
        st.run(pattern, freq)
        torch.cuda.synchronize()
        return st.idx_buf.clone(), [o.clone() for o in st.outs]

    i_def, o_def = run()
    i_f1, o_f1 = run(freq=1)
    i_all, o_all = run("F" * n)
    i_again, o_again = run()
    for a, b, c, d in zip(o_def, o_f1, o_all, o_again):
        assert torch.equal(a, b) and torch.equal(a, c) and torch.equal(a, d)
    assert torch.equal(i_def, i_f1) and torch.equal(i_def, i_again)
    pat = "FSSFSF"
    i_p, o_p = run(pat)
    for l in range(n):
        if pat[l] == "F":
            assert torch.equal(o_p[l], o_all[l]), f"F layer {l} differs from all-F"
    assert not torch.equal(o_p[1], o_all[1])
    i_f2, o_f2 = run(freq=2)
    i_p2, o_p2 = run("FSFSFS")
    for a, b in zip(o_f2, o_p2):
        assert torch.equal(a, b)
    # a rejected pattern leaves every output untouched
    before = [o.clone() for o in st.outs]
    ib = st.idx_buf.clone()
    with pytest.raises(dsa.DsaError):
        st.run("SFFFFF")
    with pytest.raises(dsa.DsaError):
        st.run("FSF")
    torch.cuda.synchronize()
    assert torch.equal(ib, st.idx_buf) and all(torch.equal(a, b) for a, b in zip(before, st.outs))


def test_stack_fp8_seeded_pattern(dsa):
    say("stack fp8")
    L, k, n = 160, 32, 5
    dev, host = _stack_layers(n, L, 64, 128, 16, 128, config=5, dtype="fp8")
    pat = seeded_pattern(n, 2, seed=5)
    st = dsa.LayerStack(dev, k)
    st.run(pat)
    torch.cuda.synchronize()
    last_f = max(l for l in range(n) if pat[l] == "F")
    _, ridx, _, _ = oracle.run_stack(host, k, pattern=pat)
    ov, _ = overlap(st.idx_buf.cpu().numpy()[0], ridx[last_f])
    assert ov >= 0.99
    for l in range(last_f, n):
        ref, _ = oracle.sparse_attention_rows(host[l]["q"], host[l]["k"], host[l]["v"],
                                              st.idx_buf.cpu().numpy()[0], range(L))
        assert np.abs(st.outs[l].float().cpu().numpy()[0] - ref).max() <= ATTN_ATOL


def test_stack_layer_events(dsa):
    dev, _ = _stack_layers(4, 128, 4, 32, 4, 64, config=1)
    st = dsa.LayerStack(dev, 16, events=True)
    st.run(freq=2)
    torch.cuda.synchronize()
    t = st.layer_times_ms()
    assert len(t) == 4 and all(x >= 0 for x in t)
