"""Decode over a paged, ragged cache, float64: the same indexer, top-k, sparse
attention and layer stack as the flat oracle, applied to each request's
logical context read out of page pools.

Layout (the usual serving-engine cache; the pages do not describe one, the
IndexCache README only runs the method inside such an engine): request b holds
L_b = clamp(seq_lens[b], 0, max_seq_len) tokens, its query is the last of them
(position L_b - 1), and token s lives at slot s % page_size of page
block_table[b, s // page_size] of a pool [num_pages, page_size, ...].

Definition followed: the logical rows X_b[s] = pool[block_table[b, s // ps],
s % ps] for s < L_b are gathered, then the flat definitions run on X_b with
pos_offset = L_b - 1. Indices are logical positions, so the IndexCache index
buffer (paper, Figure 2 caption) means the same thing as in the flat case.
Scores of positions >= L_b do not exist (-inf).
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from .attention import sparse_attention_rows
from .indexer import indexer_scores_rows, topk_from_scores
from .stack import run_stack


def request_len(seq_lens, b: int, max_seq_len: int) -> int:
    """Context length of request b, clamped into [0, max_seq_len]."""
    return int(min(max(int(np.asarray(seq_lens)[b]), 0), max_seq_len))


def gather_request(pool, block_table, b: int, n: int, page_size: int) -> np.ndarray:
    """The first n logical rows of request b: [n, ...] (same dtype as pool)."""
    pool = np.asarray(pool)
    bt = np.asarray(block_table)
    rows = [pool[int(bt[b, s // page_size]), s % page_size] for s in range(n)]
    if not rows:
        return np.zeros((0,) + pool.shape[2:], dtype=pool.dtype)
    return np.stack(rows)


def paged_indexer_topk(q_bits, k_pool, w, k: int, seq_lens, block_table, page_size: int,
                       max_seq_len: int, *, dtype: str = "bf16", q_scale=None, k_scale_pool=None):
    """q_bits [B, 1, H, D], w [B, 1, H], k_pool [num_pages, page_size, D] bits
    (k_scale_pool [num_pages, page_size] for fp8). Returns idx [B, k] int32
    (logical positions, -1 padded) and scores [B, max_seq_len] (-inf past L_b)."""
    q_bits = np.asarray(q_bits)
    B = q_bits.shape[0]
    idx = np.full((B, k), -1, dtype=np.int32)
    sc = np.full((B, max_seq_len), -np.inf)
    for b in range(B):
        n = request_len(seq_lens, b, max_seq_len)
        if n == 0:
            continue
        kb = gather_request(k_pool, block_table, b, n, page_size)[None]
        ks = None if k_scale_pool is None else gather_request(k_scale_pool, block_table, b, n, page_size)[None]
        qs = None if q_scale is None else np.asarray(q_scale)[b:b + 1]
        row = indexer_scores_rows(q_bits[b:b + 1], kb, np.asarray(w)[b:b + 1], [0], dtype=dtype,
                                  q_scale=qs, k_scale=ks, pos_offset=n - 1, batch=0)
        sc[b, :n] = row[0]
        idx[b] = topk_from_scores(row, k, pos_offset=n - 1, rows=[0])[0]
    return idx, sc


def paged_sparse_attention(q_bits, k_pool, v_pool, idx, seq_lens, block_table, page_size: int,
                           max_seq_len: int, *, scale: Optional[float] = None):
    """q_bits [B, 1, H, D] bf16 bits, k_pool / v_pool [num_pages, page_size, D],
    idx [B, topk] (or [B, 1, topk]) logical positions. Returns O [B, H, D] and
    lse [B, H]; an entry outside 0..L_b - 1 is skipped."""
    q_bits = np.asarray(q_bits)
    B, _, H, D = q_bits.shape
    I = np.asarray(idx).reshape(B, -1)
    O = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = request_len(seq_lens, b, max_seq_len)
        if n == 0:
            continue
        kb = gather_request(k_pool, block_table, b, n, page_size)[None]
        vb = gather_request(v_pool, block_table, b, n, page_size)[None]
        o, l = sparse_attention_rows(q_bits[b:b + 1], kb, vb, I[b:b + 1], [0], scale=scale,
                                     pos_offset=n - 1, batch=0)
        O[b], lse[b] = o[0], l[0]
    return O, lse


def paged_run_stack(layers: List[dict], topk: int, seq_lens, block_table, page_size: int, max_seq_len: int,
                    *, pattern: Optional[str] = None, freq: int = 0, scale: Optional[float] = None):
    """One decode step of the layer stack. layers[l] holds q_idx [B, 1, H_I, D_I],
    w, q_scale [B, 1] (fp8), q [B, 1, H, D] bits and the pools k_idx, k_scale,
    k, v. Returns (pattern, idx [n_layers][B, topk], O [n_layers][B, H, D],
    lse [n_layers][B, H])."""
    B = np.asarray(layers[0]["q"]).shape[0]
    n_layers = len(layers)
    idxs = [np.full((B, topk), -1, dtype=np.int32) for _ in range(n_layers)]
    outs = [np.zeros(np.asarray(layers[0]["q"]).shape[:1] + np.asarray(layers[0]["q"]).shape[2:])
            for _ in range(n_layers)]
    lses = [np.full((B, np.asarray(layers[0]["q"]).shape[2]), -np.inf) for _ in range(n_layers)]
    P = None
    for b in range(B):
        n = request_len(seq_lens, b, max_seq_len)
        flat = []
        for L in layers:
            g = lambda name: gather_request(L[name], block_table, b, n, page_size)[None]
            d = dict(dtype=L["dtype"], q_idx=np.asarray(L["q_idx"])[b:b + 1], w=np.asarray(L["w"])[b:b + 1],
                     q=np.asarray(L["q"])[b:b + 1], k_idx=g("k_idx"), k=g("k"), v=g("v"))
            if L.get("q_scale") is not None:
                d["q_scale"] = np.asarray(L["q_scale"])[b:b + 1]
                d["k_scale"] = g("k_scale")
            flat.append(d)
        P, ib, ob, lb = run_stack(flat, topk, pattern=pattern, freq=freq, pos_offset=n - 1, scale=scale)
        for l in range(n_layers):
            idxs[l][b], outs[l][b], lses[l][b] = ib[l][0], ob[l][0], lb[l][0]
    return P, idxs, outs, lses


def paged_append(pool, src, seq_lens, block_table, page_size: int, max_seq_len: int) -> np.ndarray:
    """A copy of pool with src[b] written at position L_b - 1 of request b
    (requests with L_b = 0 untouched)."""
    out = np.array(pool, copy=True)
    bt = np.asarray(block_table)
    for b in range(np.asarray(src).shape[0]):
        n = request_len(seq_lens, b, max_seq_len)
        if n > 0:
            s = n - 1
            out[int(bt[b, s // page_size]), s % page_size] = np.asarray(src)[b]
    return out
