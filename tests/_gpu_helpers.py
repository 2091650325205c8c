"""Shared helpers for the GPU parity tests (comparison against the CPU oracle)."""
import numpy as np
import torch

import oracle
from dsa_inputs import host_bits

SCORE_ATOL = 1e-2
SCORE_RTOL = 2e-2
ATTN_ATOL = 2e-2


def say(msg):
    print(msg, flush=True)


def run_indexer(dsa, inp, topk, dump=True, out_scores=True):
    g = inp.to("cuda")
    r = dsa.indexer_scores_topk(g.q, g.k, g.w, topk, q_scale=g.q_scale, k_scale=g.k_scale,
                                pos_offset=g.pos_offset, out_scores=out_scores,
                                debug_full_scores=dump)
    torch.cuda.synchronize()
    return r


def overlap(gpu_idx, ref_idx):
    """Aggregate set overlap sum|A & B| / sum|B| over rows (-1 entries ignored)."""
    inter = tot = 0
    worst = 1.0
    for a, b in zip(gpu_idx, ref_idx):
        sb = set(int(x) for x in b if x >= 0)
        sa = set(int(x) for x in a if x >= 0)
        inter += len(sa & sb)
        tot += len(sb)
        if sb:
            worst = min(worst, len(sa & sb) / len(sb))
    return (inter / tot if tot else 1.0), worst


def host_inputs(inp):
    return dict(q=host_bits(inp.q), k=host_bits(inp.k), w=host_bits(inp.w),
                qs=host_bits(inp.q_scale), ks=host_bits(inp.k_scale), dtype=inp.dtype,
                off=inp.pos_offset)


def check_indexer(dsa, inp, topk, *, rows=None, exact=False, min_overlap=0.99, dump=True):
    """Runs the GPU indexer and checks, for the given rows of every batch entry:
    scores (dump) vs oracle, the oracle's selection on the GPU's own scores ==
    GPU idx bitwise, out_scores == dump[idx] bitwise, and overlap (or exact
    equality) with the oracle's independent selection."""
    B, n_q, n_k, H, D = inp.shape
    r = run_indexer(dsa, inp, topk, dump=dump)
    h = host_inputs(inp)
    rows = list(range(n_q)) if rows is None else list(rows)
    ridx = torch.tensor(rows, device="cuda", dtype=torch.long)
    gidx = r.idx[:, ridx].cpu().numpy()
    gsc = r.scores[:, ridx].cpu().numpy()
    full = r.full_scores[:, ridx].cpu().numpy() if dump else None
    stats = []
    for b in range(B):
        ref = oracle.indexer_scores_rows(h["q"], h["k"], h["w"], rows, dtype=h["dtype"],
                                         q_scale=h["qs"], k_scale=h["ks"], pos_offset=h["off"],
                                         batch=b)
        causal = ref != -np.inf
        ref_idx = oracle.topk_from_scores(ref, topk, pos_offset=h["off"], rows=rows)
        if dump:
            g = full[b].astype(np.float64)
            assert np.all(np.isnan(g[~causal])), "kernel wrote a non-causal score"
            assert np.all(np.isfinite(g[causal])), "missing or non-finite causal score"
            if exact:
                assert np.array_equal(g[causal], ref[causal]), "exact-arithmetic scores differ"
            else:
                err = np.abs(g[causal] - ref[causal])
                bad = err > SCORE_ATOL + SCORE_RTOL * np.abs(ref[causal])
                assert not bad.any(), f"{bad.sum()} scores out of tolerance, max err {err.max()}"
            sel = oracle.topk_from_scores(np.where(causal, g, -np.inf), topk, pos_offset=h["off"],
                                          rows=rows)
            assert np.array_equal(sel, gidx[b]), "idx differs from the oracle's selection on GPU scores"
            valid = gidx[b] >= 0
            picked = np.take_along_axis(full[b], np.where(valid, gidx[b], 0), axis=1)
            assert np.array_equal(picked[valid].view(np.uint32), gsc[b][valid].view(np.uint32))
            assert np.all(gsc[b][~valid] == -np.inf)
        if exact:
            assert np.array_equal(ref_idx, gidx[b]), "idx differs from the oracle (exact inputs)"
            ov = (1.0, 1.0)
        else:
            ov = overlap(gidx[b], ref_idx)
            assert ov[0] >= min_overlap, f"overlap {ov}"
        # structural properties at any size
        for i, t in enumerate(rows):
            n_t = min(topk, h["off"] + t + 1, n_k)
            row = gidx[b, i]
            assert np.all(row[n_t:] == -1)
            v = row[:n_t]
            assert np.all((v >= 0) & (v <= h["off"] + t)) and len(set(v.tolist())) == n_t
            s = gsc[b, i, :n_t]
            assert np.all(np.diff(s) <= 0), "scores not in rank order"
            tie = np.diff(s) == 0
            assert np.all(np.diff(v)[tie] > 0), "ties not by lower index"
        stats.append(ov)
    return r, stats
