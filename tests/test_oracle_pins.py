"""Pins of the CPU oracle against things other than itself (runs without a GPU).

Each pin is a function of an implementation, so that the same pin is run on the
oracle (must pass) and on deliberately broken variants of it (must fail): this
shows that a plausible slip (a dropped ReLU, a misplaced weight, a causal
off-by-one, a reversed tie rule, a missing scale, a transposed operand) is
caught by at least one pin.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from dsa_inputs import make_indexer_inputs, make_int_indexer_inputs, host_bits, make_attn_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits(arr):
    return host_bits(torch.tensor(arr, dtype=torch.float32).to(torch.bfloat16))


# ---------------------------------------------------------------- implementations
class OracleImpl:
    """The oracle, seen through the interface the pins use."""

    @staticmethod
    def scores(q, k, w, rows, **kw):
        return oracle.indexer_scores_rows(q, k, w, rows, **kw)

    @staticmethod
    def topk(scores, k, pos_offset=0, rows=None):
        return oracle.topk_from_scores(scores, k, pos_offset=pos_offset, rows=rows)


def _mutant(**bugs):
    """An oracle variant with one planted mistake (CPU only, for pin sensitivity)."""

    class M(OracleImpl):
        @staticmethod
        def scores(q, k, w, rows, dtype="bf16", q_scale=None, k_scale=None, pos_offset=0,
                   batch=0):
            from oracle.formats import bf16_to_f64, e4m3fn_to_f64
            if dtype == "bf16":
                Q, K = bf16_to_f64(q[batch]), bf16_to_f64(k[batch])
            else:
                Q = e4m3fn_to_f64(q[batch]) * np.asarray(q_scale, np.float64)[batch][:, None, None]
                K = e4m3fn_to_f64(k[batch])
                if not bugs.get("drop_k_scale"):
                    K = K * np.asarray(k_scale, np.float64)[batch][:, None]
            W = np.asarray(w, np.float64)[batch]
            n_k = K.shape[0]
            out = np.full((len(rows), n_k), -np.inf)
            for r, t in enumerate(rows):
                p = pos_offset + t
                n = min(p + (0 if bugs.get("strict_causal") else 1), n_k)
                if n <= 0:
                    continue
                X = Q[t] @ K[:n].T
                if bugs.get("transpose_ts"):   # score matrix built transposed: q of row s, key t
                    X = np.stack([Q[s] @ K[t] for s in range(n)], axis=1)
                if bugs.get("drop_relu"):
                    out[r, :n] = W[t] @ X
                elif bugs.get("relu_after_weight"):
                    out[r, :n] = np.maximum(W[t][:, None] * X, 0).sum(0)
                elif bugs.get("head0_weight"):
                    out[r, :n] = W[t, 0] * np.maximum(X, 0).sum(0)
                else:
                    out[r, :n] = W[t] @ np.maximum(X, 0)
            return out

        @staticmethod
        def topk(scores, k, pos_offset=0, rows=None):
            S = np.asarray(scores, np.float64)
            R, n_k = S.shape
            rows = list(range(R)) if rows is None else list(rows)
            out = np.full((R, k), -1, np.int32)
            for r in range(R):
                n = min(pos_offset + rows[r] + 1, n_k)
                cand = np.arange(n)
                if bugs.get("ties_high_index"):
                    order = np.lexsort((-cand, -S[r, :n]))
                elif bugs.get("ascending"):
                    order = np.lexsort((cand, S[r, :n]))
                else:
                    order = np.lexsort((cand, -S[r, :n]))
                out[r, :min(k, n)] = cand[order[:min(k, n)]]
            return out

    return M


MUTANTS = {
    "drop_relu": _mutant(drop_relu=True),
    "relu_after_weight": _mutant(relu_after_weight=True),
    "head0_weight": _mutant(head0_weight=True),
    "strict_causal": _mutant(strict_causal=True),
    "ties_high_index": _mutant(ties_high_index=True),
    "ascending": _mutant(ascending=True),
    "drop_k_scale": _mutant(drop_k_scale=True),
    "transpose_ts": _mutant(transpose_ts=True),
}


# ---------------------------------------------------------------- pins
def pin_golden(impl):
    g = _load("indexer_tiny.json")
    q = _bf16_bits([g["q"]])
    k = _bf16_bits([g["k"]])
    w = np.array([g["w"]], np.float32)
    S = impl.scores(q, k, w, range(3))
    for t in range(3):
        for s in range(3):
            exp = g["scores"][t][s]
            if exp is None:
                assert S[t, s] == -np.inf
            else:
                assert S[t, s] == exp, (t, s, S[t, s], exp)
    idx = impl.topk(S, g["topk"])
    assert idx.tolist() == g["idx"]


def _as_lists(bits_q, bits_k, w, b=0):
    Q = torch.from_numpy(bits_q[b].view(np.int16)).view(torch.bfloat16).double().tolist()
    K = torch.from_numpy(bits_k[b].view(np.int16)).view(torch.bfloat16).double().tolist()
    return Q, K, np.asarray(w, np.float64)[b].tolist()


def pin_bruteforce(impl):
    cases = [  # (n_q, n_k, H, D, k, pos_offset)
        (12, 12, 3, 8, 5, 0),
        (9, 9, 4, 4, 20, 0),      # k >= L
        (10, 10, 2, 6, 1, 0),     # k = 1
        (5, 14, 3, 8, 4, 9),      # queries are the last 5 of 14 tokens
        (1, 17, 4, 8, 6, 16),     # one decode query
    ]
    for i, (n_q, n_k, H, D, k, off) in enumerate(cases):
        inp = make_indexer_inputs(1, n_q, n_k, H, D, config=90, layer=i, pos_offset=off)
        qb, kb, w = host_bits(inp.q), host_bits(inp.k), host_bits(inp.w)
        S = impl.scores(qb, kb, w, range(n_q), pos_offset=off)
        Q, K, W = _as_lists(qb, kb, w)
        ref = brute.brute_scores(Q, K, W, pos_offset=off)
        for (t, s), v in ref.items():
            assert abs(S[t, s] - v) <= 1e-12 * (1 + abs(v)), (i, t, s)
        for t in range(n_q):
            for s in range(n_k):
                if s > off + t:
                    assert S[t, s] == -np.inf
        idx = impl.topk(S, k, pos_offset=off)
        assert idx.tolist() == brute.brute_topk(ref, n_q, n_k, k, pos_offset=off), i


def pin_exact_integer(impl):
    """Integer q, k and dyadic w: brute force in exact rationals; the float64
    oracle must agree exactly, including the tie order (many ties)."""
    inp = make_int_indexer_inputs(1, 24, 24, 4, 8, seed=3)
    qb, kb, w = host_bits(inp.q), host_bits(inp.k), host_bits(inp.w)
    Q, K, W = _as_lists(qb, kb, w)
    Qf = [[[Fraction(int(x)) for x in h] for h in row] for row in Q]
    Kf = [[Fraction(int(x)) for x in r] for r in K]
    Wf = [[Fraction(x) for x in r] for r in W]
    ref = brute.brute_scores(Qf, Kf, Wf)
    S = impl.scores(qb, kb, w, range(24))
    for (t, s), v in ref.items():
        assert Fraction(S[t, s]) == v, (t, s)
    n_ties = sum(1 for t in range(24) for s in range(t) for s2 in range(s)
                 if ref[(t, s)] == ref[(t, s2)])
    assert n_ties > 20
    assert impl.topk(S, 6).tolist() == brute.brute_topk(ref, 24, 24, 6)


def pin_positive_closed_form(impl):
    """All inputs positive -> every ReLU is the identity, so the score is a plain
    GEMM: I[t,s] = (sum_j w[t,j] q[t,j,:]) . k[s,:]."""
    g = torch.Generator().manual_seed(5)
    q = torch.rand(1, 8, 3, 16, generator=g).to(torch.bfloat16)
    k = torch.rand(1, 8, 16, generator=g).to(torch.bfloat16)
    w = torch.randn(1, 8, 3, generator=g)
    S = impl.scores(host_bits(q), host_bits(k), host_bits(w), range(8))
    qw = torch.einsum("th,thc->tc", w[0].double(), q[0].double())
    ref = torch.mm(qw, k[0].double().T).numpy()
    for t in range(8):
        np.testing.assert_allclose(S[t, :t + 1], ref[t, :t + 1], rtol=1e-12, atol=1e-12)
    # one head, unit weight: the score is ReLU(q.k) of that head alone
    g2 = torch.Generator().manual_seed(6)
    q1 = torch.randn(1, 6, 1, 5, generator=g2).to(torch.bfloat16)
    k1 = torch.randn(1, 6, 5, generator=g2).to(torch.bfloat16)
    S1 = impl.scores(host_bits(q1), host_bits(k1), np.ones((1, 6, 1), np.float32), range(6))
    dots = torch.mm(q1[0, :, 0].double(), k1[0].double().T).clamp_min(0).numpy()
    for t in range(6):
        np.testing.assert_allclose(S1[t, :t + 1], dots[t, :t + 1], rtol=1e-12, atol=1e-15)


def pin_fp8_homogeneity(impl):
    """Scale homogeneity: scores(q8, k8, qs, ks)[t,s] = qs[t]*ks[s]*scores(q8, k8, 1, 1)[t,s],
    because qs, ks > 0 and ReLU is positively homogeneous."""
    inp = make_indexer_inputs(1, 10, 10, 4, 16, config=91, dtype="fp8")
    qb, kb, w = host_bits(inp.q), host_bits(inp.k), host_bits(inp.w)
    qs, ks = host_bits(inp.q_scale), host_bits(inp.k_scale)
    S = impl.scores(qb, kb, w, range(10), dtype="fp8", q_scale=qs, k_scale=ks)
    S1 = impl.scores(qb, kb, w, range(10), dtype="fp8", q_scale=np.ones_like(qs),
                     k_scale=np.ones_like(ks))
    for t in range(10):
        exp = qs[0, t].astype(np.float64) * ks[0, :t + 1].astype(np.float64) * S1[t, :t + 1]
        np.testing.assert_allclose(S[t, :t + 1], exp, rtol=1e-12, atol=1e-12)


def pin_ties_and_short_rows(impl):
    """All scores equal (q = 0) -> each row lists its first min(k, p+1) tokens in
    index order; rows with p+1 <= k hold exactly their causal tokens."""
    q = np.zeros((1, 7, 2, 4), np.uint16)
    inp = make_indexer_inputs(1, 7, 7, 2, 4, config=92)
    S = impl.scores(q, host_bits(inp.k), host_bits(inp.w), range(7))
    assert np.all(S[np.isfinite(S)] == 0)
    idx = impl.topk(S, 4)
    for t in range(7):
        n = min(4, t + 1)
        assert idx[t, :n].tolist() == list(range(n))
        assert np.all(idx[t, n:] == -1)
    S2 = impl.scores(host_bits(inp.q), host_bits(inp.k), host_bits(inp.w), range(7))
    idx2 = impl.topk(S2, 4)
    for t in range(3):
        assert sorted(idx2[t, :t + 1].tolist()) == list(range(t + 1))
        assert np.all(idx2[t, t + 1:] == -1)
        vals = S2[t, idx2[t, :t + 1]]
        assert np.all(np.diff(vals) <= 0)


PINS = [pin_golden, pin_bruteforce, pin_exact_integer, pin_positive_closed_form,
        pin_fp8_homogeneity, pin_ties_and_short_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    pin(OracleImpl)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    impl = MUTANTS[name]
    failures = 0
    for pin in PINS:
        try:
            pin(impl)
        except Exception:  # any failure of the pin counts as catching the mistake
            failures += 1
    assert failures >= 1, f"no pin catches the planted mistake {name}"


# ---------------------------------------------------------------- formats
def test_e4m3_table_matches_library_and_format():
    tab = oracle.e4m3fn_table()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(tab), nan)
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(tab[~nan], lib[~nan])
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0
    assert tab[0x01] == 2.0 ** -9 and tab[0x38] == 1.0


def test_bf16_decode_matches_library():
    g = torch.Generator().manual_seed(11)
    bits = torch.randint(0, 65536, (4096,), generator=g, dtype=torch.int32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].to(torch.int16)  # skip inf/nan codes
    ref = bits.view(torch.bfloat16).double().numpy()
    got = oracle.bf16_to_f64(bits.numpy().view(np.uint16))
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- attention
def test_attention_golden():
    g = _load("attention_tiny.json")
    q = _bf16_bits([[[g["q"]]]])         # [1, 1, 1, 2]
    k = _bf16_bits([g["k"]])
    v = _bf16_bits([g["v"]])
    idx = np.array([[g["idx"]]], np.int32)
    O, lse = oracle.sparse_attention_rows(q, k, v, idx, [0], scale=g["scale"], pos_offset=g["pos"])
    np.testing.assert_allclose(O[0, 0], g["out"], rtol=1e-13)
    assert abs(lse[0, 0] - g["lse"]) < 1e-13


def _dense_causal_sdpa(q_bits, k_bits, v_bits, scale):
    """Textbook dense causal attention with torch's SDPA in float64 (the library
    routine), one KV head broadcast to every query head."""
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).double()[0]  # [L,H,D]
    k = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16).double()[0]  # [L,D]
    v = torch.from_numpy(v_bits.view(np.int16)).view(torch.bfloat16).double()[0]
    H = q.shape[1]
    qh = q.permute(1, 0, 2)                       # [H, L, D]
    kh = k.unsqueeze(0).expand(H, -1, -1).contiguous()
    vh = v.unsqueeze(0).expand(H, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, is_causal=True, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("scale", [None, 0.3])
def test_attention_full_selection_is_dense_causal(scale):
    L, H, D = 20, 3, 16
    a = make_attn_inputs(1, L, L, H, D, config=93)
    qb, kb, vb = host_bits(a.q), host_bits(a.k), host_bits(a.v)
    rng = np.random.default_rng(0)
    idx = np.full((1, L, L + 3), -1, np.int32)
    for t in range(L):
        idx[0, t, :t + 1] = rng.permutation(t + 1)   # all causal keys, any order
    O, _ = oracle.sparse_attention(qb, kb, vb, idx, scale=scale)
    ref = _dense_causal_sdpa(qb, kb, vb, scale if scale else 1 / math.sqrt(D))
    np.testing.assert_allclose(O[0], ref, rtol=1e-10, atol=1e-12)


def test_attention_special_cases():
    L, H, D = 9, 2, 8
    a = make_attn_inputs(1, L, L, H, D, config=94)
    kb, vb = host_bits(a.k), host_bits(a.v)
    V = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).double().numpy()[0]
    K = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).double().numpy()[0]
    zero_q = np.zeros((1, L, H, D), np.uint16)
    idx = np.array([[[0, 3, 5, -1]] * L], np.int32)
    O, lse = oracle.sparse_attention_rows(zero_q, kb, vb, idx, [8])
    np.testing.assert_allclose(O[0, 0], V[[0, 3, 5]].mean(0), rtol=1e-13)  # q = 0: mean of V
    assert abs(lse[0, 0] - math.log(3)) < 1e-13                            # lse = log n
    qb = host_bits(a.q)
    one = np.array([[[4, -1, -1, -1]] * L], np.int32)
    O1, lse1 = oracle.sparse_attention_rows(qb, kb, vb, one, [6])
    np.testing.assert_allclose(O1[0, 1], V[4], rtol=1e-15)               # one key: its V row
    Q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).double().numpy()[0]
    assert abs(lse1[0, 1] - Q[6, 1] @ K[4] / math.sqrt(D)) < 1e-12
    # out-of-range (non-causal) entries are skipped; an empty selection gives 0, -inf
    bad = np.array([[[7, 8, -1, -1]] * L], np.int32)
    O2, lse2 = oracle.sparse_attention_rows(qb, kb, vb, bad, [2])
    assert np.all(O2 == 0) and np.all(lse2 == -np.inf)


def test_attention_matches_bruteforce():
    L, H, D, k = 11, 2, 6, 4
    a = make_attn_inputs(1, L, L, H, D, config=95)
    qb, kb, vb = host_bits(a.q), host_bits(a.k), host_bits(a.v)
    rng = np.random.default_rng(1)
    idx = np.full((1, L, k), -1, np.int32)
    for t in range(L):
        n = min(k, t + 1)
        idx[0, t, :n] = rng.choice(t + 1, n, replace=False)
    O, lse = oracle.sparse_attention(qb, kb, vb, idx, scale=0.7)
    tq = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().tolist()
    Q, K, V = tq(qb)[0], tq(kb)[0], tq(vb)[0]
    for t in range(L):
        sel = [int(i) for i in idx[0, t] if i >= 0]
        for h in range(H):
            o, l = brute.brute_attention(Q[t][h], K, V, sel, 0.7)
            np.testing.assert_allclose(O[0, t, h], o, rtol=1e-12, atol=1e-14)
            assert abs(lse[0, t, h] - l) < 1e-12
