"""GPU parity of dsa_indexer_scores_topk against the CPU oracle (prefill and decode)."""
import numpy as np
import pytest
import torch

from dsa_inputs import make_indexer_inputs, make_int_indexer_inputs
from _gpu_helpers import check_indexer, overlap, run_indexer, say

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ prefill
@pytest.mark.parametrize("shape,topk", [
    ((1, 256, 256, 4, 32), 16),      # tiny stack layer shape
    ((1, 300, 300, 64, 128), 64),    # two head blocks, ragged last tile
    ((2, 97, 97, 20, 64), 8),        # heads not a multiple of 32, B = 2
])
def test_prefill_exact_integer(dsa, shape, topk):
    say(f"prefill exact {shape} k={topk}")
    inp = make_int_indexer_inputs(*shape, seed=11)
    check_indexer(dsa, inp, topk, exact=True)


@pytest.mark.parametrize("shape,topk,cfg", [
    ((1, 256, 256, 4, 32), 16, 1),
    ((1, 1000, 1000, 64, 128), 64, 2),     # many in-kernel compactions (list capacity 576)
    ((1, 333, 333, 64, 64), 300, 3),       # k close to L
    ((1, 2, 2, 64, 128), 16, 4),           # smallest prefill
    ((1, 130, 700, 64, 128), 32, 5),       # chunked prefill: queries are the last 130 of 700
])
def test_prefill_random_bf16(dsa, shape, topk, cfg):
    say(f"prefill bf16 {shape} k={topk}")
    inp = make_indexer_inputs(*shape, config=cfg)
    check_indexer(dsa, inp, topk)


@pytest.mark.parametrize("L", [63, 64, 65, 127, 128, 129, 191, 255, 257])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefill_tile_boundaries(dsa, L, dtype):
    """Lengths around the 64-key sub-tile and 128-key iteration boundaries
    (rows of one workgroup ending in different sub-tiles, a last sub-tile
    wholly past the keys)."""
    say(f"prefill {dtype} L={L}")
    inp = make_indexer_inputs(1, L, L, 16, 64, config=11, dtype=dtype)
    check_indexer(dsa, inp, 24)


def test_prefill_small_k_many_shrinks(dsa):
    """k = 8 over 3000 keys: the list (capacity k + 512) is shrunk over and over."""
    say("prefill k=8 L=3000")
    inp = make_indexer_inputs(1, 3000, 3000, 32, 64, config=12)
    rows = [0, 7, 8, 519, 520, 521, 1500, 2999] + list(np.random.default_rng(1).choice(3000, 24, replace=False))
    check_indexer(dsa, inp, 8, rows=sorted(set(int(r) for r in rows)))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefill_k2048_compaction(dsa, dtype):
    """k = 2048 with rows longer than the 8192-entry candidate list (4k), so the
    in-kernel shrink runs (first when a list nears 8192 - 256 entries); sampled
    rows incl. the first shrinking ones and the capacity boundary."""
    L = 9000
    say(f"prefill {dtype} L={L} k=2048")
    inp = make_indexer_inputs(1, L, L, 64, 128, config=6, w_std=0.125, dtype=dtype)
    rows = [0, 1, 2046, 2047, 2048, 2049, 7870, 7935, 7936, 7937, 8000, 8191, 8192, 8193, L - 2, L - 1]
    rows += list(np.random.default_rng(0).choice(L, 25, replace=False))
    check_indexer(dsa, inp, 2048, rows=sorted(set(int(r) for r in rows)))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefill_scores_across_zero_wide_range(dsa, dtype):
    """Exact inputs whose keys are scaled by 2^-12, except every 61st by 2^5:
    every row's scores take both signs, almost all of them tiny, a few large.
    Rows holding every causal key bucket a range across zero (by the score,
    not the key bits), whose middle bucket then overflows: the ranking must
    fall back to the exact select. Rows past 1.5 k candidates go through the
    narrowing pre-pass first. Scores stay exact: each one's terms share the
    key's scale."""
    say(f"prefill {dtype} scores across zero, wide range")
    L = 4000
    inp = make_int_indexer_inputs(1, L, L, 16, 64, seed=21, dtype=dtype)
    scale = torch.full((L,), 2.0 ** -12)
    scale[::61] = 2.0 ** 5
    if dtype == "bf16":
        inp.k = (inp.k.float() * scale[None, :, None]).to(torch.bfloat16)
    else:
        inp.k_scale = (inp.k_scale * scale[None, :]).contiguous()
    rows = [0, 1, 60, 61, 62, 2046, 2047, 2048, 3070, 3071, 3072, 3073, L - 1]
    rows += list(np.random.default_rng(3).choice(L, 12, replace=False))
    check_indexer(dsa, inp, 2048, rows=sorted(set(int(r) for r in rows)), exact=True)


def test_prefill_all_ties(dsa):
    """q = 0: every score is 0, so each row must list its first min(k, t+1)
    tokens in index order (tie rule through many compactions)."""
    say("prefill all ties")
    inp = make_indexer_inputs(1, 700, 700, 8, 64, config=7)
    inp.q.zero_()
    r, _ = check_indexer(dsa, inp, 64, exact=True)
    idx = r.idx.cpu().numpy()[0]
    for t in (0, 5, 63, 64, 699):
        n = min(64, t + 1)
        assert idx[t, :n].tolist() == list(range(n))


@pytest.mark.parametrize("exact", [True, False])
def test_prefill_fp8(dsa, exact):
    say(f"prefill fp8 exact={exact}")
    if exact:
        inp = make_int_indexer_inputs(1, 300, 300, 64, 128, seed=12, dtype="fp8")
    else:
        inp = make_indexer_inputs(1, 300, 300, 64, 128, config=8, dtype="fp8")
    check_indexer(dsa, inp, 64, exact=exact)


def test_prefill_fp8_d64(dsa):
    say("prefill fp8 D=64")
    inp = make_indexer_inputs(1, 200, 200, 16, 64, config=9, dtype="fp8")
    check_indexer(dsa, inp, 32)


def test_prefill_dump_mode_does_not_change_result(dsa):
    inp = make_indexer_inputs(1, 600, 600, 64, 128, config=10)
    a = run_indexer(dsa, inp, 128, dump=True)
    b = run_indexer(dsa, inp, 128, dump=False)
    c = run_indexer(dsa, inp, 128, dump=False)
    assert torch.equal(a.idx, b.idx) and torch.equal(b.idx, c.idx)
    assert torch.equal(a.scores.view(torch.int32), b.scores.view(torch.int32))


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("B,n_k,topk,cfg", [
    (3, 5000, 2048, 20),
    (1, 777, 64, 21),
    (2, 100, 2048, 22),   # fewer keys than k: -1 padding
])
def test_decode_random_bf16(dsa, B, n_k, topk, cfg):
    say(f"decode bf16 B={B} n_k={n_k} k={topk}")
    inp = make_indexer_inputs(B, 1, n_k, 64, 128, config=cfg, w_std=0.125)
    check_indexer(dsa, inp, topk)


def test_decode_weights_4byte_aligned(dsa):
    """w need only be 4-byte aligned: a w that starts 4 bytes into its
    allocation (its rows then not 16-byte aligned although H % 4 == 0) gives
    bitwise the same selection and scores as an aligned copy."""
    say("decode w at a 4-byte offset")
    B, n_k, H, k = 3, 5000, 64, 512
    inp = make_indexer_inputs(B, 1, n_k, H, 128, config=23, w_std=0.125).to("cuda")
    store = torch.empty(B * H + 1, dtype=torch.float32, device="cuda")
    w_off = store[1:].view(B, 1, H)
    w_off.copy_(inp.w)
    assert w_off.data_ptr() % 16 == 4
    a = dsa.indexer_scores_topk(inp.q, inp.k, inp.w, k, out_scores=True)
    b = dsa.indexer_scores_topk(inp.q, inp.k, w_off, k, out_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(a.idx, b.idx)
    assert torch.equal(a.scores.view(torch.int32), b.scores.view(torch.int32))


def test_decode_exact_integer(dsa):
    say("decode exact")
    inp = make_int_indexer_inputs(2, 1, 3000, 64, 128, seed=13)
    check_indexer(dsa, inp, 100, exact=True)


@pytest.mark.parametrize("n_k,topk,qk,H,D", [
    (9000, 2048, 3, 64, 128),   # hundreds of short runs of equal scores among the winners
    (6000, 512, 1, 16, 32),     # a run longer than 32: re-sort with index passes (16-bit indices)
    (70000, 2048, 1, 4, 32),    # the same with indices above 65535
])
def test_decode_tie_runs(dsa, n_k, topk, qk, H, D):
    """Exact-integer scores with many equal values among the top-k but no list
    overflow: equal scores must come out in index order."""
    say(f"decode tie runs n_k={n_k} k={topk}")
    inp = make_int_indexer_inputs(1, 1, n_k, H, D, seed=13, qk_range=qk)
    check_indexer(dsa, inp, topk, exact=True)


def test_decode_all_ties_overflow_path(dsa):
    """All scores equal: the candidate list overflows and the exact full-row
    select must return the k lowest indices in order."""
    say("decode all ties")
    inp = make_indexer_inputs(1, 1, 9000, 64, 128, config=23)
    inp.q.zero_()
    r, _ = check_indexer(dsa, inp, 2048, exact=True)
    assert r.idx.cpu().numpy()[0, 0].tolist() == list(range(2048))


def test_decode_dense_threshold_bin(dsa):
    """Every key in one 12-bit histogram bin, so the candidate list holds all
    6000 keys (more than half its 8192-entry capacity): the ranking path with
    its second batch of entries, nearly all scores distinct."""
    say("decode dense bin")
    inp = make_indexer_inputs(2, 1, 6000, 16, 128, config=25)
    g = torch.Generator().manual_seed(5)
    # scores 11.5 +- 0.1: inside [11, 12), one bin of the top 12 order-key bits
    inp.k.copy_((1.0 + 0.02 * torch.randn(inp.k.shape, generator=g)).to(inp.k.dtype))
    inp.q.copy_((0.0898 + 0.002 * torch.randn(inp.q.shape, generator=g)).to(inp.q.dtype))
    inp.w.fill_(1.0 / 16)
    r, _ = check_indexer(dsa, inp, 2048)
    full = r.full_scores.cpu().numpy()
    assert np.all(full > 11.0) and np.all(full < 12.0)


def test_decode_all_ties_within_capacity(dsa):
    """All 6000 scores equal with the list inside its capacity: one bucket
    exceeds the ranking path's run limit and the sort path takes over; the
    tie rule gives the first k indices."""
    say("decode all ties, list within capacity")
    inp = make_indexer_inputs(1, 1, 6000, 64, 128, config=26)
    inp.q.zero_()
    r, _ = check_indexer(dsa, inp, 2048, exact=True)
    assert r.idx.cpu().numpy()[0, 0].tolist() == list(range(2048))


def test_decode_fp8(dsa):
    say("decode fp8")
    inp = make_indexer_inputs(2, 1, 4000, 64, 128, config=24, dtype="fp8")
    check_indexer(dsa, inp, 512)


@pytest.mark.parametrize("L,topk,H,D", [(3000, 8, 4, 32), (9000, 2048, 16, 64)])
def test_prefill_every_key_accepted(dsa, L, topk, H, D):
    """score(t, s) = H * s exactly (q = (256, 1, 0, ..), k_s = (s // 256,
    s % 256, 0, ..), w = 1), rising with the key index: every key passes the
    row's threshold, so each commit appends the most it can and the list is
    flagged and shrunk as often as the list margin allows. Each row's top-k
    is its k latest keys, newest first."""
    say(f"prefill every key accepted L={L} k={topk}")
    inp = make_int_indexer_inputs(1, L, L, H, D, seed=14)
    inp.q.zero_()
    inp.q[..., 0] = 256
    inp.q[..., 1] = 1
    s = torch.arange(L)
    inp.k.zero_()
    inp.k[0, :, 0] = (s // 256).to(inp.k.dtype)
    inp.k[0, :, 1] = (s % 256).to(inp.k.dtype)
    inp.w.fill_(1.0)
    rows = [0, 1, topk - 1, topk, topk + 1, L // 2, L - 2, L - 1]
    rows += list(np.random.default_rng(3).choice(L, 24, replace=False))
    r, _ = check_indexer(dsa, inp, topk, rows=sorted(set(int(x) for x in rows)), exact=True)
    t = np.arange(L)[:, None]
    j = np.arange(topk)[None, :]
    assert np.array_equal(r.idx.cpu().numpy()[0], np.where(t - j >= 0, t - j, -1))


@pytest.mark.parametrize("shape,topk,cfg", [
    ((1, 130, 700, 64, 128), 32, 15),     # chunked prefill: queries are the last 130 of 700
    ((2, 333, 333, 64, 128), 100, 16),    # two batch entries
    ((1, 129, 1000, 16, 64), 200, 17),    # d = 64, chunk ending in a ragged tile
])
def test_prefill_fp8_chunked_and_batched(dsa, shape, topk, cfg):
    say(f"prefill fp8 {shape} k={topk}")
    inp = make_indexer_inputs(*shape, config=cfg, dtype="fp8")
    check_indexer(dsa, inp, topk)
