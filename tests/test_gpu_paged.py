"""GPU parity of the paged, ragged decode entry points (dsa_paged_*): against
the paged oracle, and bitwise against the flat entry points on the same logical
data (a key's score and an entry's attention weight do not depend on where its
row lives, so paging must not change a single bit)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import paged as OP
from dsa_inputs import (host_bits, make_attn_inputs, make_indexer_inputs, make_paged_layout, randn,
                        scatter_to_pages, to_e4m3_clipped)
from _gpu_helpers import ATTN_ATOL, SCORE_ATOL, SCORE_RTOL, overlap, say

pytestmark = pytest.mark.gpu


def _junk(shape, dtype, seed):
    x = randn(shape, seed) * 4
    if dtype == torch.float8_e4m3fn:
        return to_e4m3_clipped(x)
    if dtype == torch.float32:
        return x.abs() + 0.5
    return x.to(dtype)


def _paged_indexer(dsa, lens, page_size, max_len, topk, dtype, cfg, H=64, D=128):
    B = len(lens)
    lay = make_paged_layout(lens, page_size, max_len, seed=cfg)
    inp = make_indexer_inputs(B, 1, max_len, H, D, config=cfg, dtype=dtype, w_std=0.125)
    kp = scatter_to_pages(inp.k, lay, _junk((lay.num_pages, page_size, D), inp.k.dtype, cfg + 1))
    sp = None
    if dtype == "fp8":
        sp = scatter_to_pages(inp.k_scale, lay, _junk((lay.num_pages, page_size), torch.float32, cfg + 2))
    g = inp.to("cuda")
    gl = lay.to("cuda")
    kv = dsa.PagedKV(gl.seq_lens, gl.block_table, page_size, lay.num_pages, max_len)
    r = dsa.paged_indexer_topk(g.q, kp.cuda(), g.w, topk, kv, q_scale=g.q_scale,
                               k_scale_pool=None if sp is None else sp.cuda(), out_scores=True,
                               debug_full_scores=True)
    torch.cuda.synchronize()
    return inp, lay, kp, sp, r


def _check_against_oracle(inp, lay, kp, sp, r, topk, min_overlap=0.99):
    lens = [min(max(int(x), 0), lay.max_seq_len) for x in lay.seq_lens]
    ref_idx, ref_sc = OP.paged_indexer_topk(host_bits(inp.q), host_bits(kp), host_bits(inp.w), topk,
                                            lay.seq_lens.numpy(), lay.block_table.numpy(), lay.page_size,
                                            lay.max_seq_len, dtype=inp.dtype, q_scale=host_bits(inp.q_scale),
                                            k_scale_pool=host_bits(sp))
    gidx = r.idx.cpu().numpy()[:, 0]
    gsc = r.scores.cpu().numpy()[:, 0]
    full = r.full_scores.cpu().numpy()[:, 0]
    for b, n in enumerate(lens):
        g = full[b].astype(np.float64)
        assert np.all(np.isnan(g[n:])), f"request {b}: score written past its length {n}"
        assert np.all(np.isfinite(g[:n]))
        err = np.abs(g[:n] - ref_sc[b, :n])
        assert not (err > SCORE_ATOL + SCORE_RTOL * np.abs(ref_sc[b, :n])).any(), f"request {b}: max err {err.max()}"
        # the oracle's selection on the GPU's own scores == the GPU's indices
        sel = oracle.topk_from_scores(np.where(np.arange(lay.max_seq_len) < n, g, -np.inf)[None], topk,
                                      pos_offset=n - 1)[0]
        assert np.array_equal(sel, gidx[b]), f"request {b} (len {n}): idx differs from the oracle's selection"
        n_t = min(topk, n)
        assert np.all(gidx[b, n_t:] == -1) and np.all(gsc[b, n_t:] == -np.inf)
        if n_t:
            assert np.array_equal(full[b][gidx[b, :n_t]].view(np.uint32), gsc[b, :n_t].view(np.uint32))
        ov, _ = overlap(gidx[b:b + 1], ref_idx[b:b + 1])
        assert ov >= min_overlap, f"request {b}: overlap {ov}"


@pytest.mark.parametrize("lens,page_size,max_len,topk,dtype,cfg", [
    ([1, 63, 64, 65, 3000, 0, 5000, 2049], 64, 5000, 2048, "bf16", 70),
    ([4000, 33, 129], 32, 4000, 512, "fp8", 71),
    ([700, 12000, 1], 256, 12000, 2048, "bf16", 72),     # one long request among short ones
])
def test_paged_indexer_ragged(dsa, lens, page_size, max_len, topk, dtype, cfg):
    say(f"paged indexer lens={lens} page={page_size} k={topk} {dtype}")
    inp, lay, kp, sp, r = _paged_indexer(dsa, lens, page_size, max_len, topk, dtype, cfg)
    _check_against_oracle(inp, lay, kp, sp, r, topk)


def test_paged_indexer_many_requests(dsa):
    """More requests than the planning block has threads (each thread plans
    several), empty ones among them, a single page each or many."""
    say("paged indexer B=300")
    rng = np.random.default_rng(76)
    lens = rng.integers(0, 3000, size=300).tolist()
    lens[:3] = [0, 1, 2999]
    inp, lay, kp, sp, r = _paged_indexer(dsa, lens, 32, 3000, 64, "bf16", 76, H=16, D=64)
    _check_against_oracle(inp, lay, kp, sp, r, 64)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_indexer_equals_flat(dsa, dtype):
    """Every request at full length, pages shuffled: bitwise the flat result."""
    say(f"paged == flat indexer {dtype}")
    B, L, topk = 3, 4096, 2048
    inp, lay, kp, sp, r = _paged_indexer(dsa, [L] * B, 128, L, topk, dtype, 73)
    g = inp.to("cuda")
    f = dsa.indexer_scores_topk(g.q, g.k, g.w, topk, q_scale=g.q_scale, k_scale=g.k_scale, pos_offset=L - 1,
                                out_scores=True, debug_full_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(r.idx, f.idx)
    assert torch.equal(r.scores.view(torch.int32), f.scores.view(torch.int32))
    assert torch.equal(r.full_scores.view(torch.int32), f.full_scores.view(torch.int32))


def test_paged_indexer_ragged_equals_flat_per_request(dsa):
    """A request of length n over the pool == the flat call over its n keys."""
    say("paged ragged == flat per request")
    lens, topk = [300, 2500, 64], 256
    inp, lay, kp, sp, r = _paged_indexer(dsa, lens, 32, 2500, topk, "bf16", 74)
    for b, n in enumerate(lens):
        q = inp.q[b:b + 1].cuda()
        k = inp.k[b:b + 1, :n].contiguous().cuda()
        w = inp.w[b:b + 1].cuda()
        f = dsa.indexer_scores_topk(q, k, w, topk, pos_offset=n - 1, out_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(r.idx[b], f.idx[0]), f"request {b}"
        assert torch.equal(r.scores[b].view(torch.int32), f.scores[0].view(torch.int32))


def test_paged_indexer_no_debug_dump_same_result(dsa):
    lens, topk = [900, 17, 2000], 512
    inp, lay, kp, sp, r = _paged_indexer(dsa, lens, 64, 2000, topk, "bf16", 75)
    g, gl = inp.to("cuda"), lay.to("cuda")
    kv = dsa.PagedKV(gl.seq_lens, gl.block_table, 64, lay.num_pages, 2000)
    r2 = dsa.paged_indexer_topk(g.q, kp.cuda(), g.w, topk, kv, out_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(r.idx, r2.idx)
    assert torch.equal(r.scores.view(torch.int32), r2.scores.view(torch.int32))


# ------------------------------------------------------------------ attention
def _paged_attn_case(lens, page_size, max_len, H, D, cfg):
    B = len(lens)
    lay = make_paged_layout(lens, page_size, max_len, seed=cfg)
    a = make_attn_inputs(B, 1, max_len, H, D, config=cfg)
    kp = scatter_to_pages(a.k, lay, _junk((lay.num_pages, page_size, D), torch.bfloat16, cfg + 1))
    vp = scatter_to_pages(a.v, lay, _junk((lay.num_pages, page_size, D), torch.bfloat16, cfg + 2))
    return a, lay, kp, vp


def _ragged_idx(lens, topk, seed, junk=True):
    rng = np.random.default_rng(seed)
    idx = np.full((len(lens), 1, topk), -1, np.int32)
    for b, n in enumerate(lens):
        n = max(n, 0)
        m = min(topk, n)
        if m:
            idx[b, 0, :m] = rng.choice(n, m, replace=False)
        if junk and topk > m + 1:
            idx[b, 0, m] = n + int(rng.integers(0, 5))   # past the request's end: skipped
    return idx


@pytest.mark.parametrize("lens,page_size,max_len,H,D,topk,cfg", [
    ([1, 63, 64, 65, 3000, 0, 5000], 64, 5000, 16, 128, 2048, 80),
    ([200, 4096], 32, 4096, 12, 64, 512, 81),   # H < 16, D = 64
])
def test_paged_attn_ragged(dsa, lens, page_size, max_len, H, D, topk, cfg):
    say(f"paged attn lens={lens} H={H} D={D} k={topk}")
    a, lay, kp, vp = _paged_attn_case(lens, page_size, max_len, H, D, cfg)
    idx = _ragged_idx(lens, topk, cfg)
    gl = lay.to("cuda")
    kv = dsa.PagedKV(gl.seq_lens, gl.block_table, page_size, lay.num_pages, max_len)
    out, lse = dsa.paged_sparse_attn(a.q.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(idx).cuda(), kv, lse=True)
    torch.cuda.synchronize()
    O = out.float().cpu().numpy()[:, 0]
    LS = lse.cpu().numpy()[:, 0]
    ref_o, ref_l = OP.paged_sparse_attention(host_bits(a.q), host_bits(kp), host_bits(vp), idx,
                                             lay.seq_lens.numpy(), lay.block_table.numpy(), page_size, max_len)
    err = np.abs(O - ref_o).max()
    assert err <= ATTN_ATOL, f"max-abs error {err}"
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(LS))
    assert np.abs(LS[fin] - ref_l[fin]).max() <= 1e-3 * (1 + np.abs(ref_l[fin]).max())
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(O[b] == 0) and np.all(LS[b] == -np.inf)


def test_paged_attn_equals_flat(dsa):
    say("paged == flat attn")
    B, L, topk = 4, 5000, 2048
    a, lay, kp, vp = _paged_attn_case([L] * B, 64, L, 16, 128, 82)
    idx = torch.from_numpy(_ragged_idx([L] * B, topk, 82)).cuda()
    gl = lay.to("cuda")
    kv = dsa.PagedKV(gl.seq_lens, gl.block_table, 64, lay.num_pages, L)
    g = a.to("cuda")
    o1, l1 = dsa.paged_sparse_attn(g.q, kp.cuda(), vp.cuda(), idx, kv, lse=True)
    o2, l2 = dsa.sparse_attn(g.q, g.k, g.v, idx, pos_offset=L - 1, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


# ------------------------------------------------------------------ append
@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (128, torch.float8_e4m3fn), (1, torch.float32)])
def test_paged_append_rows(dsa, D, dtype):
    say(f"paged append D={D} {dtype}")
    lens = [1, 64, 65, 0, 300, 128]
    lay = make_paged_layout(lens, 64, 300, seed=90)
    shape = (lay.num_pages, 64) + ((D,) if D > 1 else ())
    pool = _junk(shape, dtype, 91)
    src = _junk((len(lens),) + shape[2:], dtype, 92)
    gl = lay.to("cuda")
    kv = dsa.PagedKV(gl.seq_lens, gl.block_table, 64, lay.num_pages, 300)
    gp = pool.cuda()
    dsa.paged_append_rows(src.cuda(), gp, kv)
    torch.cuda.synchronize()
    ref = OP.paged_append(host_bits(pool), host_bits(src), lay.seq_lens.numpy(), lay.block_table.numpy(), 64, 300)
    assert np.array_equal(host_bits(gp), ref)


# ------------------------------------------------------------------ stack
def _paged_stack(dsa, lens, page_size, max_len, n_layers, cfg, dtype="bf16", H_I=64, D_I=128, H=16, D=128):
    B = len(lens)
    lay = make_paged_layout(lens, page_size, max_len, seed=cfg)
    gl = lay.to("cuda")
    kv = dsa.PagedKV(gl.seq_lens, gl.block_table, page_size, lay.num_pages, max_len)
    flat, paged, host = [], [], []
    for l in range(n_layers):
        ii = make_indexer_inputs(B, 1, max_len, H_I, D_I, config=cfg, layer=l, dtype=dtype, w_std=0.125)
        aa = make_attn_inputs(B, 1, max_len, H, D, config=cfg, layer=l)
        pools = {}
        for nm, t, s in (("k_idx", ii.k, 1), ("k", aa.k, 2), ("v", aa.v, 3)):
            pools[nm] = scatter_to_pages(t, lay, _junk((lay.num_pages, page_size, t.shape[-1]), t.dtype,
                                                       cfg * 100 + 10 * l + s))
        if dtype == "fp8":
            pools["k_scale"] = scatter_to_pages(ii.k_scale, lay, _junk((lay.num_pages, page_size), torch.float32,
                                                                       cfg * 100 + 10 * l + 4))
        g, ga = ii.to("cuda"), aa.to("cuda")
        flat.append(dict(q_idx=g.q, k_idx=g.k, w=g.w, q_scale=g.q_scale, k_scale=g.k_scale, q=ga.q, k=ga.k, v=ga.v))
        paged.append(dict(q_idx=g.q, k_idx=pools["k_idx"].cuda(), w=g.w, q_scale=g.q_scale,
                          k_scale=pools["k_scale"].cuda() if dtype == "fp8" else None,
                          q=ga.q, k=pools["k"].cuda(), v=pools["v"].cuda()))
        host.append(dict(dtype=dtype, q_idx=host_bits(ii.q), w=host_bits(ii.w), q=host_bits(aa.q),
                         q_scale=host_bits(ii.q_scale),
                         k_scale=host_bits(pools.get("k_scale")),
                         k_idx=host_bits(pools["k_idx"]), k=host_bits(pools["k"]), v=host_bits(pools["v"])))
    return lay, kv, flat, paged, host


def test_paged_stack_equals_flat_and_separate_calls(dsa):
    say("paged stack == flat stack")
    n, L, k = 4, 3000, 2048
    lay, kv, flat, paged, _ = _paged_stack(dsa, [L] * 3, 64, L, n, 95)
    sp = dsa.LayerStack(paged, k, lse=True, kv=kv)
    sf = dsa.LayerStack(flat, k, lse=True)
    for pat in ("FSFS", None, "FSSS"):
        sp.run(pat)
        sf.run(pat)
        torch.cuda.synchronize()
        assert torch.equal(sp.idx_buf, sf.idx_buf)
        for a, b in zip(sp.outs, sf.outs):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the last run ("FSSS") equals a separate indexer call and separate attention calls
    r0 = dsa.paged_indexer_topk(paged[0]["q_idx"], paged[0]["k_idx"], paged[0]["w"], k, kv)
    torch.cuda.synchronize()
    assert torch.equal(r0.idx, sp.idx_buf)
    for l in range(n):
        o, _ = dsa.paged_sparse_attn(paged[l]["q"], paged[l]["k"], paged[l]["v"], r0.idx, kv)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), sp.outs[l].view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_stack_ragged_vs_oracle(dsa, dtype):
    say(f"paged stack ragged {dtype}")
    lens, n, k = [1000, 0, 37, 2600], 3, 512
    lay, kv, _, paged, host = _paged_stack(dsa, lens, 32, 2600, n, 96, dtype=dtype)
    st = dsa.LayerStack(paged, k, lse=True, kv=kv)
    st.run("FSF")
    torch.cuda.synchronize()
    P, ridx, _, _ = OP.paged_run_stack(host, k, lay.seq_lens.numpy(), lay.block_table.numpy(), 32, 2600,
                                       pattern="FSF")
    gidx = st.idx_buf.cpu().numpy()[:, 0]
    ov, _ = overlap(gidx, ridx[2])
    assert ov >= 0.99, f"overlap {ov}"
    # the last layer's attention over the GPU's own indices vs the oracle
    O, _ = OP.paged_sparse_attention(host[2]["q"], host[2]["k"], host[2]["v"], gidx, lay.seq_lens.numpy(),
                                     lay.block_table.numpy(), 32, 2600)
    err = np.abs(st.outs[2].float().cpu().numpy()[:, 0] - O).max()
    assert err <= ATTN_ATOL, f"max-abs error {err}"
    assert np.all(gidx[1] == -1) and torch.all(st.outs[2][1] == 0)
