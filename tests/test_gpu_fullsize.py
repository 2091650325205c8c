"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (no debug dump in the timed call).

At sizes where the oracle cannot score every pair, the checks are:
  * properties that hold at any size, checked on every row on the GPU
    (range, padding, no duplicates, rank order, tie order);
  * sampled row blocks re-run through the same kernel as chunked prefill
    (n_q = 8 with a position offset) in test mode with the full score dump:
    their indices must equal the full run's bit for bit, the oracle's
    selection on those GPU scores must reproduce them exactly, and the
    oracle's own fp64 scores / selection must agree within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import (host_bits, make_attn_inputs, make_indexer_inputs, seeded_pattern)
from _gpu_helpers import ATTN_ATOL, SCORE_ATOL, SCORE_RTOL, overlap, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _release_memory():
    """The full-size tests hold tens of GB each: hand the cached blocks back
    between them."""
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def structural(idx, scores, pos_offset, n_k):
    """Every-row properties of [R, k] GPU outputs (scores=None: index checks only)."""
    R, k = idx.shape
    dev = idx.device
    t = torch.arange(R, device=dev, dtype=torch.int64) + pos_offset
    n_t = torch.clamp(torch.clamp(t + 1, max=n_k), max=k)
    col = torch.arange(k, device=dev)
    valid = col[None, :] < n_t[:, None]
    idx64 = idx.long()
    assert bool((idx64[~valid] == -1).all()), "padding is not -1"
    assert bool(((idx64 >= 0) | ~valid).all()) and bool(((idx64 <= t[:, None]) | ~valid).all()), \
        "index out of the causal range"
    big = torch.where(valid, idx64, torch.full_like(idx64, 1 << 40) + col[None, :])
    srt = torch.sort(big, dim=1).values
    assert bool((srt[:, 1:] != srt[:, :-1]).all()), "duplicate index in a row"
    if scores is None:
        return
    both = valid[:, 1:]
    sd = scores[:, 1:] - scores[:, :-1]
    assert bool((sd[both] <= 0).all()), "scores not in rank order"
    ties = both & (sd == 0)
    assert bool(((idx64[:, 1:] - idx64[:, :-1])[ties] > 0).all()), "ties not by lower index"
    assert bool(torch.isfinite(scores[valid]).all())


def chunk_check(dsa, inp, full_idx, t0, n, topk, oracle_rows=None):
    """Re-run rows [t0, t0+n) as chunked prefill in dump mode and check them:
    the chunk's indices equal the full run's bit for bit, the oracle's selection
    on the GPU's own scores reproduces them exactly, and for the given rows of
    the block (all of them if None) the oracle's fp64 scores agree within
    tolerance. Returns (intersection, total) of the independent selections."""
    g = inp
    q = g.q[:, t0:t0 + n].contiguous()
    w = g.w[:, t0:t0 + n].contiguous()
    qs = None if g.q_scale is None else g.q_scale[:, t0:t0 + n].contiguous()
    r = dsa.indexer_scores_topk(q, g.k, w, topk, q_scale=qs, k_scale=g.k_scale, pos_offset=t0,
                                out_scores=True, debug_full_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(r.idx[0], full_idx[0, t0:t0 + n]), f"chunk [{t0},{t0+n}) differs from the full run"
    n_k = g.k.shape[1]
    kk = min(n_k, t0 + n)
    dump = r.full_scores[0, :, :kk].cpu().numpy().astype(np.float64)
    gidx = r.idx[0].cpu().numpy()
    gsc = r.scores[0].cpu().numpy()
    causal = np.arange(kk)[None, :] <= (t0 + np.arange(n))[:, None]
    assert np.all(np.isfinite(dump[causal]))
    sel = oracle.topk_from_scores(np.where(causal, dump, -np.inf), topk, pos_offset=t0)
    assert np.array_equal(sel, gidx), "oracle selection on GPU scores differs"
    valid = gidx >= 0
    picked = np.take_along_axis(r.full_scores[0, :, :kk].cpu().numpy(), np.where(valid, gidx, 0), axis=1)
    assert np.array_equal(picked[valid].view(np.uint32), gsc[valid].view(np.uint32)), "out_scores != dump[idx]"
    h = dict(q=host_bits(q), w=host_bits(w), qs=host_bits(qs))
    kh = _host_keys(g)
    rows = list(range(n)) if oracle_rows is None else sorted(set(oracle_rows))
    ref = oracle.indexer_scores_rows(h["q"], kh[0], h["w"], rows, dtype=g.dtype, q_scale=h["qs"],
                                     k_scale=kh[1], pos_offset=t0)[:, :kk]
    for i, rr in enumerate(rows):
        c = causal[rr]
        err = np.abs(dump[rr][c] - ref[i][c])
        assert np.all(err <= SCORE_ATOL + SCORE_RTOL * np.abs(ref[i][c])), f"row {t0 + rr}: max err {err.max()}"
    ref_idx = oracle.topk_from_scores(ref, topk, pos_offset=t0, rows=rows)
    inter = tot = 0
    for a, b in zip(gidx[rows], ref_idx):
        sb = set(int(x) for x in b if x >= 0)
        inter += len(set(int(x) for x in a if x >= 0) & sb)
        tot += len(sb)
    return inter, tot


def _host_keys(g):
    """Host bits of a layer's keys (and key scales), copied once per inputs object."""
    if "_host_k" not in g.__dict__:
        g.__dict__["_host_k"] = (host_bits(g.k), host_bits(g.k_scale))
    return g.__dict__["_host_k"]


def special_chunks(L, topk, seed, n_seeded=4, n=8):
    """Starts of n-row blocks that cover t in {0, 1, k-2, k-1, k, k+1, L-1}
    plus n_seeded seeded random blocks (at least 8 blocks = 64 rows)."""
    starts = [0, topk - 8, topk, L - n]
    rng = np.random.default_rng(seed)
    while len(starts) < 4 + n_seeded:
        t0 = int(rng.integers(topk + n, L - 2 * n))
        if all(abs(t0 - s) >= n for s in starts):
            starts.append(t0)
    return sorted(starts)


def test_c2_prefill_10240_full(dsa):
    """L = 10240, H_I = 64, d_I = 128, k = 2048, bf16: the oracle's selection on
    the GPU's scores is checked on every row; fp64 oracle scores on 256 rows."""
    L, topk = 10240, 2048
    say("C2 full")
    inp = make_indexer_inputs(1, L, L, 64, 128, config=2, w_std=0.125).to("cuda")
    r = dsa.indexer_scores_topk(inp.q, inp.k, inp.w, topk, out_scores=True, debug_full_scores=True)
    r2 = dsa.indexer_scores_topk(inp.q, inp.k, inp.w, topk, out_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(r.idx, r2.idx) and torch.equal(r.scores.view(torch.int32), r2.scores.view(torch.int32))
    structural(r.idx[0], r.scores[0], 0, L)
    dump = r.full_scores[0].cpu().numpy()
    gidx = r.idx[0].cpu().numpy()
    sel = oracle.topk_from_scores(np.where(np.arange(L)[None, :] <= np.arange(L)[:, None], dump, -np.inf)
                                  .astype(np.float64), topk)
    assert np.array_equal(sel, gidx), "oracle selection on GPU scores differs"
    rows = sorted(set([0, 1, 2046, 2047, 2048, 4095, 4096, 8191, L - 1] +
                      np.random.default_rng(1).choice(L, 247, replace=False).tolist()))
    h = dict(q=host_bits(inp.q), k=host_bits(inp.k), w=host_bits(inp.w))
    ref = oracle.indexer_scores_rows(h["q"], h["k"], h["w"], rows)
    g = dump[rows].astype(np.float64)
    causal = ref != -np.inf
    err = np.abs(g[causal] - ref[causal])
    assert np.all(err <= SCORE_ATOL + SCORE_RTOL * np.abs(ref[causal])), f"max err {err.max()}"
    ov = overlap(gidx[rows], oracle.topk_from_scores(ref, topk, rows=rows))
    say(f"C2 overlap {ov}")
    assert ov[0] >= 0.99


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_prefill_200k(dsa, dtype):
    """The 200K-token layer (fp8 e4m3 with per-token scales, and bf16), full run
    as benchmarked, every-row properties; 8 blocks of 8 rows (t in {0, 1, k-2,
    k-1, k, k+1, L-1} and seeded rows: 64 rows) re-run with the dump, every one
    of those rows checked against the fp64 oracle."""
    L, topk = 200000, 2048
    say(f"200K {dtype}")
    inp = make_indexer_inputs(1, L, L, 64, 128, config=5, dtype=dtype, w_std=0.125, device="cuda")
    r = dsa.indexer_scores_topk(inp.q, inp.k, inp.w, topk, q_scale=inp.q_scale, k_scale=inp.k_scale,
                                out_scores=True)
    torch.cuda.synchronize()
    structural(r.idx[0], r.scores[0], 0, L)
    inter = tot = 0
    starts = special_chunks(L, topk, seed=5_000_017)
    for t0 in starts:
        say(f"200K {dtype} block {t0}")
        a, b = chunk_check(dsa, inp, r.idx, t0, 8, topk)
        inter, tot = inter + a, tot + b
    say(f"200K {dtype}: {8 * len(starts)} oracle rows, overlap {inter / tot:.5f}")
    assert 8 * len(starts) >= 64
    assert inter / tot >= 0.99


def _c3_layer(l, L, dev="cuda"):
    ii = make_indexer_inputs(1, L, L, 64, 128, config=3, layer=l, w_std=0.125, device=dev)
    aa = make_attn_inputs(1, L, L, 16, 128, config=3, layer=l, device=dev)
    return ii, aa


@pytest.mark.timeout(900)
def test_c3_stack_61440_freq4(dsa):
    """47 layers at L = 61440 (indexer H_I=64 d_I=128 k=2048; attention 16
    heads d=128 one KV head), index_topk_freq = 4 vs all-F. Two F layers (0 and
    44) are checked against the fp64 oracle on 64 rows each (t in {0, 1, k-2,
    k-1, k, k+1, L-1} and seeded rows), re-run with the dump."""
    L, topk, n = 61440, 2048, 47
    say("C3 stack")
    layers, inps = [], []
    for l in range(n):
        ii, aa = _c3_layer(l, L)
        inps.append(ii)
        layers.append(dict(q_idx=ii.q, k_idx=ii.k, w=ii.w, q_scale=None, k_scale=None, q=aa.q, k=aa.k, v=aa.v))
    st = dsa.LayerStack(layers, topk)
    st.run(freq=4)
    torch.cuda.synchronize()
    P = dsa.resolve_pattern(n, None, 4)
    last_f = max(l for l in range(n) if P[l] == "F")
    assert last_f == 44
    idx_f = st.idx_buf.clone()
    outs = {l: st.outs[l].clone() for l in (1, 2, 3, 43, 44, 45, 46)}
    structural(idx_f[0], None, 0, L)
    # the cached buffer is layer 44's own selection
    own = dsa.indexer_scores_topk(layers[44]["q_idx"], layers[44]["k_idx"], layers[44]["w"], topk)
    own0 = dsa.indexer_scores_topk(layers[0]["q_idx"], layers[0]["k_idx"], layers[0]["w"], topk)
    torch.cuda.synchronize()
    assert torch.equal(own.idx, idx_f)
    # S layers attend over the preceding F layer's indices, bit for bit
    for l, src in ((1, own0), (2, own0), (3, own0), (45, own), (46, own)):
        o, _ = dsa.sparse_attn(layers[l]["q"], layers[l]["k"], layers[l]["v"], src.idx)
        torch.cuda.synchronize()
        assert torch.equal(o, outs[l]), f"S layer {l} did not reuse its F layer's indices"
    # F layers 0 and 44 against the oracle on 64 rows each
    for l, full in ((0, own0.idx), (44, idx_f)):
        inter = tot = 0
        for t0 in special_chunks(L, topk, seed=3_000_017 + l):
            say(f"C3 layer {l} block {t0}")
            a, b = chunk_check(dsa, inps[l], full, t0, 8, topk)
            inter, tot = inter + a, tot + b
        say(f"C3 layer {l}: overlap {inter / tot:.5f}")
        assert inter / tot >= 0.99
    # layers 44..46 attended over it; check sampled rows against the oracle
    rows = [0, 1, 2047, 2048, 30000, L - 1]
    gi = idx_f[0].cpu().numpy()
    for l in (44, 45, 46):
        a = layers[l]
        ka, va = host_bits(a["k"]), host_bits(a["v"])
        # one oracle call per row, at the row's true position
        ref = np.stack([oracle.sparse_attention_rows(host_bits(a["q"][:, [t]]), ka, va, gi[[t]], [0],
                                                     pos_offset=t)[0][0]
                        for t in rows])
        got = outs[l][0, rows].float().cpu().numpy()
        assert np.abs(got - ref).max() <= ATTN_ATOL, f"layer {l}"
    # layer 43 is S and reuses layer 40's selection: it differs from 44's
    st.run()  # all-F
    torch.cuda.synchronize()
    assert torch.equal(st.outs[44], outs[44]), "an F layer differs between all-F and freq 4"
    assert not torch.equal(st.outs[45], outs[45]), "reuse is not equality (layer 45)"


def _check_decode_layer(dsa, ii, r, topk, T, B, tag):
    """Every request of one decode F layer against the fp64 oracle: scores
    within tolerance over all T keys, the oracle's selection on the GPU's scores
    equal to the GPU's indices, out_scores == dump[idx], and >= 99% overlap with
    the oracle's own selection."""
    kh = host_bits(ii.k)
    qh, wh = host_bits(ii.q), host_bits(ii.w)
    gidx = r.idx.cpu().numpy()
    gsc = r.scores.cpu().numpy()
    dump = r.full_scores.cpu().numpy()
    inter = tot = 0
    worst = 1.0
    for b in range(B):
        ref = oracle.indexer_scores_rows(qh, kh, wh, [0], pos_offset=T - 1, batch=b)
        err = np.abs(dump[b].astype(np.float64) - ref)
        assert np.all(err <= SCORE_ATOL + SCORE_RTOL * np.abs(ref)), f"{tag} request {b}: max err {err.max()}"
        sel = oracle.topk_from_scores(dump[b].astype(np.float64), topk, pos_offset=T - 1)
        assert np.array_equal(sel, gidx[b]), f"{tag} request {b}: oracle selection on GPU scores differs"
        picked = dump[b, 0, gidx[b, 0]]
        assert np.array_equal(picked.view(np.uint32), gsc[b, 0].view(np.uint32)), f"{tag} request {b}"
        ov = overlap(gidx[b], oracle.topk_from_scores(ref, topk, pos_offset=T - 1))
        inter += ov[0] * topk
        tot += topk
        worst = min(worst, ov[1])
    say(f"{tag}: overlap {inter / tot:.5f} (worst request {worst:.5f})")
    assert inter / tot >= 0.99
    return kh


@pytest.mark.timeout(900)
@pytest.mark.parametrize("B", [1, 32])
def test_c4_decode_stack_200k(dsa, B):
    """Decode: B single-token queries, each over its own 200000-token cache, on
    the seeded 12-F 47-layer pattern. The stack runs through its second F layer
    (and the S layer after it); both F layers are checked against the oracle on
    every request, and every S layer's output equals attention over its F
    layer's indices bit for bit."""
    T, topk, n = 200000, 2048, 47
    pat = seeded_pattern(n, 12, seed=1_000_000 * 4 + 9)
    fl = [l for l in range(n) if pat[l] == "F"][:2]
    n_run = fl[1] + 2
    say(f"C4 decode stack B={B}: pattern {pat}, F layers {fl}, {n_run} layers run")
    inps, attns, layers = [], [], []
    for l in range(n_run):
        ii = make_indexer_inputs(B, 1, T, 64, 128, config=4, layer=l, w_std=0.125, device="cuda")
        aa = make_attn_inputs(B, 1, T, 16, 128, config=4, layer=l, device="cuda")
        inps.append(ii)
        attns.append(aa)
        layers.append(dict(q_idx=ii.q, k_idx=ii.k, w=ii.w, q_scale=None, k_scale=None, q=aa.q, k=aa.k, v=aa.v))
    st = dsa.LayerStack(layers, topk)
    st.run(pat[:n_run])
    torch.cuda.synchronize()
    res = {}
    for f in fl:
        say(f"C4 B={B} F layer {f}")
        res[f] = dsa.indexer_scores_topk(inps[f].q, inps[f].k, inps[f].w, topk, out_scores=True,
                                         debug_full_scores=True)
        torch.cuda.synchronize()
        for b in range(B):
            structural(res[f].idx[b], res[f].scores[b], T - 1, T)
    assert torch.equal(st.idx_buf, res[fl[1]].idx), "the stack's cached buffer is not its last F layer's"
    for l in range(n_run):
        src = res[max(f for f in fl if f <= l)].idx
        o, _ = dsa.sparse_attn(layers[l]["q"], layers[l]["k"], layers[l]["v"], src)
        torch.cuda.synchronize()
        if not torch.equal(o, st.outs[l]):
            diff = (o.float() - st.outs[l].float()).abs().amax(dim=(1, 2, 3))
            bad = torch.nonzero(diff).flatten().tolist()
            raise AssertionError(f"layer {l} ({pat[l]}) did not attend over its F layer's indices: requests {bad} "
                                 f"differ, max abs {diff.max().item()}")
    for f in fl:
        _check_decode_layer(dsa, inps[f], res[f], topk, T, B, f"C4 B={B} layer {f}")
    # attention against the oracle: the F layer and the S layer after it, a few requests
    for l in (fl[1], fl[1] + 1):
        gidx = res[fl[1]].idx.cpu().numpy()
        for b in sorted(set([0, B - 1])):
            a = attns[l]
            ref_o, _ = oracle.sparse_attention_rows(host_bits(a.q[b:b + 1]), host_bits(a.k[b:b + 1]),
                                                    host_bits(a.v[b:b + 1]), gidx[b], [0], pos_offset=T - 1)
            err = np.abs(st.outs[l][b].float().cpu().numpy() - ref_o).max()
            assert err <= ATTN_ATOL, f"layer {l} request {b}: attention max-abs error {err}"


@pytest.mark.parametrize("B", [4, 32])
def test_c4_decode_200k(dsa, B):
    """Decode at T = 200000 outside a stack: every request against the oracle
    (B = 4 and the benchmarked B = 32)."""
    T, topk = 200000, 2048
    say(f"C4 decode B={B}")
    ii = make_indexer_inputs(B, 1, T, 64, 128, config=4, w_std=0.125, device="cuda")
    aa = make_attn_inputs(B, 1, T, 16, 128, config=4, device="cuda")
    r = dsa.indexer_scores_topk(ii.q, ii.k, ii.w, topk, out_scores=True, debug_full_scores=True)
    out, lse = dsa.sparse_attn(aa.q, aa.k, aa.v, r.idx, lse=True)
    torch.cuda.synchronize()
    for b in range(B):
        structural(r.idx[b], r.scores[b], T - 1, T)
    _check_decode_layer(dsa, ii, r, topk, T, B, f"C4 B={B}")
    gidx = r.idx.cpu().numpy()
    for b in sorted(set([0, 1, B - 1])):
        ref_o, ref_l = oracle.sparse_attention_rows(host_bits(aa.q[b:b + 1]), host_bits(aa.k[b:b + 1]),
                                                    host_bits(aa.v[b:b + 1]), gidx[b], [0], pos_offset=T - 1)
        assert np.abs(out[b].float().cpu().numpy() - ref_o).max() <= ATTN_ATOL


@pytest.mark.timeout(900)
def test_c5_stack_200k_quarter_f(dsa):
    """The 47-layer L = 200000 stack with the fp8 indexer and the seeded 12-F
    pattern, as benchmarked (one shared output buffer). The cached buffer after
    the run is the last F layer's own selection, the last (S) layer attended
    over it bit for bit, and that F layer matches the fp64 oracle on sampled
    rows; a run of the first three layers ("FSS") checks that both S layers
    reuse layer 0's indices."""
    L, topk, n = 200000, 2048, 47
    pat = seeded_pattern(n, 12, seed=1_000_000 * 5 + 9)
    last_f = max(l for l in range(n) if pat[l] == "F")
    assert pat[:3] == "FSS" and pat[-1] == "S"
    say(f"C5 stack: pattern {pat}, last F layer {last_f}")
    layers, inps = [], []
    for l in range(n):
        ii = make_indexer_inputs(1, L, L, 64, 128, config=5, layer=l, dtype="fp8", w_std=0.125, device="cuda")
        aa = make_attn_inputs(1, L, L, 16, 128, config=5, layer=l, device="cuda")
        inps.append(ii)
        layers.append(dict(q_idx=ii.q, k_idx=ii.k, w=ii.w, q_scale=ii.q_scale, k_scale=ii.k_scale,
                           q=aa.q, k=aa.k, v=aa.v))
    st = dsa.LayerStack(layers, topk, shared_out=True)
    st.run(pat)
    torch.cuda.synchronize()
    say("C5 stack ran")
    f = inps[last_f]
    own = dsa.indexer_scores_topk(f.q, f.k, f.w, topk, q_scale=f.q_scale, k_scale=f.k_scale)
    torch.cuda.synchronize()
    assert torch.equal(own.idx, st.idx_buf), "cached buffer is not the last F layer's selection"
    o, _ = dsa.sparse_attn(layers[-1]["q"], layers[-1]["k"], layers[-1]["v"], own.idx)
    torch.cuda.synchronize()
    assert torch.equal(o, st.outs[-1]), "the last S layer did not attend over the cached indices"
    structural(st.idx_buf[0], None, 0, L)
    inter = tot = 0
    for t0 in (0, topk - 8, L - 8):
        say(f"C5 stack layer {last_f} block {t0}")
        a, b = chunk_check(dsa, f, st.idx_buf, t0, 8, topk)
        inter, tot = inter + a, tot + b
    assert inter / tot >= 0.99
    del st
    torch.cuda.empty_cache()
    # the first three layers with their own outputs: S layers 1 and 2 reuse layer 0
    st3 = dsa.LayerStack(layers[:3], topk)
    st3.run(pat[:3])
    f0 = inps[0]
    own0 = dsa.indexer_scores_topk(f0.q, f0.k, f0.w, topk, q_scale=f0.q_scale, k_scale=f0.k_scale)
    torch.cuda.synchronize()
    assert torch.equal(own0.idx, st3.idx_buf)
    for l in (0, 1, 2):
        o, _ = dsa.sparse_attn(layers[l]["q"], layers[l]["k"], layers[l]["v"], own0.idx)
        torch.cuda.synchronize()
        assert torch.equal(o, st3.outs[l]), f"layer {l} did not attend over layer 0's indices"
