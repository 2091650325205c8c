"""Pins of the paged-decode oracle (oracle/paged.py) against the flat oracle
(itself pinned elsewhere) and against layout invariants: the pool is built by
scattering flat rows (the inputs module), the oracle reads it by gathering, so a
wrong page or slot lookup, a wrong query position or a lost clamp fails here."""
import numpy as np
import pytest
import torch

import oracle
from oracle import paged as P
from dsa_inputs import host_bits, make_indexer_inputs, make_attn_inputs, make_paged_layout, scatter_to_pages, randn

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

PS = 32
MAXL = 150
LENS = [1, 31, 32, 33, 150, 0, 97]


def _paged_indexer_case(dtype, lens=LENS, seed=5):
    B = len(lens)
    lay = make_paged_layout(lens, PS, MAXL, seed=seed)
    inp = make_indexer_inputs(B, 1, MAXL, 4, 32, config=40 + seed, dtype=dtype)
    junk = randn((lay.num_pages, PS, 32), 999 + seed).to(inp.k.dtype)
    pool = scatter_to_pages(inp.k, lay, junk)
    spool = None
    if dtype == "fp8":
        spool = scatter_to_pages(inp.k_scale, lay, torch.full((lay.num_pages, PS), 3.0))
    return inp, lay, pool, spool


def _run_paged(inp, lay, pool, spool, k):
    return P.paged_indexer_topk(host_bits(inp.q), host_bits(pool), host_bits(inp.w), k, lay.seq_lens.numpy(),
                                lay.block_table.numpy(), lay.page_size, lay.max_seq_len, dtype=inp.dtype,
                                q_scale=host_bits(inp.q_scale), k_scale_pool=host_bits(spool))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_indexer_equals_flat_per_request(dtype):
    """Request b over the pool == the flat oracle over the first L_b flat keys,
    query at position L_b - 1."""
    inp, lay, pool, spool = _paged_indexer_case(dtype)
    k = 16
    idx, sc = _run_paged(inp, lay, pool, spool, k)
    h = dict(q=host_bits(inp.q), k=host_bits(inp.k), w=host_bits(inp.w), qs=host_bits(inp.q_scale),
             ks=host_bits(inp.k_scale))
    for b, n in enumerate(LENS):
        if n == 0:
            assert np.all(idx[b] == -1) and np.all(sc[b] == -np.inf)
            continue
        ref_idx, ref_sc = oracle.indexer_topk(h["q"][b:b + 1], h["k"][b:b + 1, :n], h["w"][b:b + 1], k,
                                              dtype=dtype, q_scale=None if h["qs"] is None else h["qs"][b:b + 1],
                                              k_scale=None if h["ks"] is None else h["ks"][b:b + 1, :n],
                                              pos_offset=n - 1)
        assert np.array_equal(idx[b], ref_idx[0, 0])
        assert np.array_equal(sc[b, :n], ref_sc[0, 0])
        assert np.all(sc[b, n:] == -np.inf)
        n_t = min(k, n)
        assert np.all(idx[b, n_t:] == -1) and np.all((idx[b, :n_t] >= 0) & (idx[b, :n_t] < n))


def test_paged_indexer_ignores_slots_outside_the_context():
    """Junk in unused pages and in slots at or past L_b changes nothing."""
    inp, lay, pool, _ = _paged_indexer_case("bf16")
    a = _run_paged(inp, lay, pool, None, 16)
    junk2 = randn(pool.shape, 4242).to(pool.dtype) * 50
    pool2 = scatter_to_pages(inp.k, lay, junk2)
    assert not torch.equal(pool, pool2)
    b = _run_paged(inp, lay, pool2, None, 16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_paged_indexer_page_permutation_invariance():
    """Renaming pages (pool pages permuted, block table renamed to match) gives
    identical results; renaming the table alone does not."""
    inp, lay, pool, _ = _paged_indexer_case("bf16")
    a = _run_paged(inp, lay, pool, None, 16)
    perm = np.random.default_rng(3).permutation(lay.num_pages)      # new page id of old page p: perm[p]
    pool2 = torch.empty_like(pool)
    pool2[torch.from_numpy(perm)] = pool
    bt = lay.block_table.numpy()
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    lay2 = type(lay)(lay.seq_lens, torch.from_numpy(bt2), lay.page_size, lay.num_pages, lay.max_seq_len)
    b = _run_paged(inp, lay2, pool2, None, 16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = _run_paged(inp, lay2, pool, None, 16)                          # table renamed, pool not
    assert not np.array_equal(a[1], c[1])


def test_paged_lengths_are_clamped():
    lens = [-5, MAXL + 40]
    inp, lay, pool, _ = _paged_indexer_case("bf16", lens=lens)
    idx, sc = _run_paged(inp, lay, pool, None, 8)
    assert np.all(idx[0] == -1) and np.all(sc[0] == -np.inf)
    ref_idx, ref_sc = oracle.indexer_topk(host_bits(inp.q)[1:2], host_bits(inp.k)[1:2], host_bits(inp.w)[1:2], 8,
                                          pos_offset=MAXL - 1)
    assert np.array_equal(idx[1], ref_idx[0, 0]) and np.array_equal(sc[1], ref_sc[0, 0])


def test_paged_attention_equals_flat_and_empty_request():
    lens = LENS
    B = len(lens)
    lay = make_paged_layout(lens, PS, MAXL, seed=9)
    a = make_attn_inputs(B, 1, MAXL, 4, 64, config=51)
    kp = scatter_to_pages(a.k, lay, randn((lay.num_pages, PS, 64), 77).to(torch.bfloat16))
    vp = scatter_to_pages(a.v, lay, randn((lay.num_pages, PS, 64), 78).to(torch.bfloat16))
    rng = np.random.default_rng(1)
    idx = rng.integers(-3, MAXL + 3, size=(B, 24)).astype(np.int32)   # includes -1 and past-the-end entries
    O, lse = P.paged_sparse_attention(host_bits(a.q), host_bits(kp), host_bits(vp), idx, lay.seq_lens.numpy(),
                                      lay.block_table.numpy(), PS, MAXL)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(O[b] == 0) and np.all(lse[b] == -np.inf)
            continue
        ro, rl = oracle.sparse_attention_rows(host_bits(a.q)[b:b + 1], host_bits(a.k)[b:b + 1, :n],
                                              host_bits(a.v)[b:b + 1, :n], idx[b:b + 1], [0], pos_offset=n - 1)
        assert np.array_equal(O[b], ro[0]) and np.array_equal(lse[b], rl[0])


def test_paged_append_extends_the_logical_view():
    lens = [1, 40, 64, 0, 150]
    lay = make_paged_layout(lens, PS, MAXL, seed=2)
    pool = randn((lay.num_pages, PS, 8), 5).numpy()
    src = randn((len(lens), 8), 6).numpy()
    out = P.paged_append(pool, src, lay.seq_lens.numpy(), lay.block_table.numpy(), PS, MAXL)
    changed = 0
    for b, n in enumerate(lens):
        before = P.gather_request(pool, lay.block_table.numpy(), b, n, PS)
        after = P.gather_request(out, lay.block_table.numpy(), b, n, PS)
        if n:
            assert np.array_equal(after[:n - 1], before[:n - 1]) and np.array_equal(after[n - 1], src[b])
            changed += 1
    assert (out != pool).any(axis=2).sum() == changed


def test_paged_stack_equals_flat_stack_per_request():
    lens = [40, 0, 150]
    B, n_layers, k = len(lens), 3, 8
    lay = make_paged_layout(lens, PS, MAXL, seed=4)
    layers, pooled = [], []
    for l in range(n_layers):
        ii = make_indexer_inputs(B, 1, MAXL, 4, 32, config=60, layer=l)
        aa = make_attn_inputs(B, 1, MAXL, 4, 64, config=60, layer=l)
        junk = lambda t, s: randn((lay.num_pages, PS) + tuple(t.shape[2:]), s).to(t.dtype)
        layers.append(dict(dtype="bf16", q_idx=host_bits(ii.q), k_idx=host_bits(ii.k), w=host_bits(ii.w),
                           q=host_bits(aa.q), k=host_bits(aa.k), v=host_bits(aa.v)))
        pooled.append(dict(dtype="bf16", q_idx=host_bits(ii.q), w=host_bits(ii.w), q=host_bits(aa.q),
                           k_idx=host_bits(scatter_to_pages(ii.k, lay, junk(ii.k, 100 + l))),
                           k=host_bits(scatter_to_pages(aa.k, lay, junk(aa.k, 200 + l))),
                           v=host_bits(scatter_to_pages(aa.v, lay, junk(aa.v, 300 + l)))))
    Pt, idxs, outs, lses = P.paged_run_stack(pooled, k, lay.seq_lens.numpy(), lay.block_table.numpy(), PS, MAXL,
                                             pattern="FSF")
    assert Pt == "FSF"
    for b, n in enumerate(lens):
        flat = [{key: (v[b:b + 1, :n] if key in ("k_idx", "k", "v") else
                       (v[b:b + 1] if key != "dtype" else v)) for key, v in L.items()} for L in layers]
        _, ri, ro, rl = oracle.run_stack(flat, k, pattern="FSF", pos_offset=n - 1)
        for l in range(n_layers):
            assert np.array_equal(idxs[l][b], ri[l][0])
            assert np.array_equal(outs[l][b], ro[l][0]) and np.array_equal(lses[l][b], rl[l][0])
    # the S layer reuses layer 0's indices
    assert np.array_equal(idxs[1], idxs[0])
