"""Lightning-indexer scores and per-query top-k selection, float64.

Definition followed (plain form; the fast path reaches the same result up to
rounding order):

  Dequantise. bf16: Q = q, K = k exactly. fp8 e4m3fn with per-token scales:
  Q[t,j,:] = e4m3(q[t,j,:]) * q_scale[t], K[s,:] = e4m3(k[s,:]) * k_scale[s].

  Score. Query t sits at position p(t) = pos_offset + t and sees keys
  0 <= s <= p(t) (causal, the diagonal included):
      I[t,s] = sum_j W[t,j] * max(0, sum_c Q[t,j,c] * K[s,c]).
  Entries with s > p(t) do not exist (returned as -inf).

  Top-k. n_t = min(k, p(t) + 1). The candidates 0..p(t) are ordered by score,
  higher first, equal scores by lower index first; row t lists the first n_t of
  them in that order, and is padded with -1 up to k. -0.0 and +0.0 are equal.

The IndexCache abstract describes the indexer as selecting the top-k tokens per
query for the sparse core attention; the tie rule and the padding are this
library's fixed reading (the pages leave them open).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .formats import bf16_to_f64, e4m3fn_to_f64


def _dequant(q_bits, k_bits, dtype: str, q_scale=None, k_scale=None):
    """Returns float64 Q [B, n_q, H, D] and K [B, n_k, D]."""
    if dtype == "bf16":
        return bf16_to_f64(q_bits), bf16_to_f64(k_bits)
    if dtype == "fp8":
        qs = np.asarray(q_scale, dtype=np.float64)
        ks = np.asarray(k_scale, dtype=np.float64)
        if not (np.all(qs > 0) and np.all(ks > 0)):
            raise ValueError("fp8 scales must be > 0")
        Q = e4m3fn_to_f64(q_bits) * qs[:, :, None, None]
        K = e4m3fn_to_f64(k_bits) * ks[:, :, None]
        return Q, K
    raise ValueError(f"unknown dtype {dtype}")


def indexer_scores_rows(q_bits, k_bits, w, rows: Sequence[int], *, dtype: str = "bf16",
                        q_scale=None, k_scale=None, pos_offset: int = 0,
                        batch: int = 0) -> np.ndarray:
    """Scores of the given query rows of one batch entry: [len(rows), n_k] float64,
    -inf where the key is not causal for that row."""
    rows = [int(t) for t in rows]
    # only the requested query rows are dequantised
    Q, K = _dequant(np.asarray(q_bits)[batch:batch + 1, rows], k_bits[batch:batch + 1], dtype,
                    None if q_scale is None else np.asarray(q_scale)[batch:batch + 1, rows],
                    None if k_scale is None else np.asarray(k_scale)[batch:batch + 1])
    Q = Q[0]                                   # [len(rows), H, D]
    K = K[0]
    W = np.asarray(w, dtype=np.float64)[batch]
    n_k = K.shape[0]
    out = np.full((len(rows), n_k), -np.inf)
    for r, t in enumerate(rows):
        p = pos_offset + t
        n = min(p + 1, n_k)
        if n <= 0:
            continue
        # X[j, s] = Q[t,j,:] . K[s,:]  for the causal keys of this row.
        X = Q[r] @ K[:n].T
        out[r, :n] = W[t] @ np.maximum(X, 0.0)
    if not np.all(np.isfinite(out[out != -np.inf])):
        raise ValueError("non-finite score: inputs must be finite")
    return out + 0.0  # -0.0 -> +0.0


def indexer_scores(q_bits, k_bits, w, *, dtype: str = "bf16", q_scale=None, k_scale=None,
                   pos_offset: int = 0) -> np.ndarray:
    """All scores: [B, n_q, n_k] float64 (-inf where not causal)."""
    B, n_q = np.asarray(w).shape[:2]
    n_k = np.asarray(k_bits).shape[1]
    out = np.empty((B, n_q, n_k))
    for b in range(B):
        out[b] = indexer_scores_rows(q_bits, k_bits, w, range(n_q), dtype=dtype,
                                     q_scale=q_scale, k_scale=k_scale,
                                     pos_offset=pos_offset, batch=b)
    return out


def topk_from_scores(scores, k: int, *, pos_offset: int = 0,
                     rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Top-k of each row of a score matrix [R, n_k] (row r is query rows[r], or r).
    Candidates of query t are keys 0..min(p(t), n_k - 1); returns int32 [R, k]."""
    S = np.asarray(scores, dtype=np.float64)
    R, n_k = S.shape
    rows = list(range(R)) if rows is None else list(rows)
    out = np.full((R, k), -1, dtype=np.int32)
    for r in range(R):
        p = pos_offset + int(rows[r])
        n = min(p + 1, n_k)
        if n <= 0:
            continue
        cand = np.arange(n)
        vals = S[r, :n] + 0.0
        if not np.all(np.isfinite(vals)):
            raise ValueError("non-finite score among causal candidates")
        order = np.lexsort((cand, -vals))  # primary: score descending; then index ascending
        n_t = min(k, n)
        out[r, :n_t] = cand[order[:n_t]]
    return out


def indexer_topk(q_bits, k_bits, w, k: int, *, dtype: str = "bf16", q_scale=None,
                 k_scale=None, pos_offset: int = 0, rows: Optional[Sequence[int]] = None):
    """Indices [B, R, k] int32 and scores [B, R, n_k] of the given rows (all rows
    if None) of every batch entry."""
    B, n_q = np.asarray(w).shape[:2]
    rows = list(range(n_q)) if rows is None else list(rows)
    n_k = np.asarray(k_bits).shape[1]
    idx = np.empty((B, len(rows), k), dtype=np.int32)
    sc = np.empty((B, len(rows), n_k))
    for b in range(B):
        sc[b] = indexer_scores_rows(q_bits, k_bits, w, rows, dtype=dtype, q_scale=q_scale,
                                    k_scale=k_scale, pos_offset=pos_offset, batch=b)
        idx[b] = topk_from_scores(sc[b], k, pos_offset=pos_offset, rows=rows)
    return idx, sc


def score_order_key(scores_f32) -> np.ndarray:
    """uint32 key of fp32 scores that orders like the values (higher key = higher
    score), with -0.0 mapped like +0.0. Used by tests to compare orders."""
    s = np.asarray(scores_f32, dtype=np.float32) + np.float32(0.0)
    b = s.view(np.uint32)
    neg = (b >> np.uint32(31)) == 1
    return np.where(neg, ~b, b | np.uint32(0x80000000)).astype(np.uint32)
