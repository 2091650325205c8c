"""Sparse core attention over selected token indices, float64.

Definition followed (the IndexCache abstract: the indexer's top-k selection
makes core attention cost O(L*k) instead of O(L^2); the pages do not spell the
attention out, so this is the plain softmax attention restricted to the
selected set). For query t at position p(t) = pos_offset + t, head h:

  Sel_t   = the entries r of idx[t, :] with 0 <= idx[t,r] <= p(t) and
            idx[t,r] < n_k (entries equal to -1, or otherwise out of range,
            are skipped; each valid entry counts once per occurrence)
  a_r     = scale * sum_c q[t,h,c] * K[idx[t,r], c]          (r in Sel_t)
  m       = max_r a_r
  P_r     = exp(a_r - m) / sum_r' exp(a_r' - m)
  O[t,h]  = sum_r P_r * V[idx[t,r], :]
  lse     = m + log(sum_r exp(a_r - m))

All H query heads share one K and one V head. scale defaults to 1/sqrt(D).
An empty Sel_t gives O = 0 and lse = -inf.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .formats import bf16_to_f64


def sparse_attention_rows(q_bits, k_bits, v_bits, idx, rows: Sequence[int], *,
                          scale: Optional[float] = None, pos_offset: int = 0,
                          batch: int = 0):
    """Output [len(rows), H, D] and lse [len(rows), H] (float64) of the given
    query rows of one batch entry. idx is [n_q, topk] (or [B, n_q, topk])."""
    Q = bf16_to_f64(np.asarray(q_bits)[batch])      # [n_q, H, D]
    K = bf16_to_f64(np.asarray(k_bits)[batch])      # [n_k, D]
    V = bf16_to_f64(np.asarray(v_bits)[batch])
    I = np.asarray(idx)
    if I.ndim == 3:
        I = I[batch]
    n_k, D = K.shape
    H = Q.shape[1]
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(D)
    O = np.zeros((len(rows), H, D))
    lse = np.full((len(rows), H), -np.inf)
    for r, t in enumerate(rows):
        p = pos_offset + int(t)
        sel = [int(i) for i in I[t] if 0 <= int(i) <= p and int(i) < n_k]
        if not sel:
            continue
        Ks = K[sel]                                   # [n, D]
        Vs = V[sel]
        a = scale * (Q[t] @ Ks.T)                     # [H, n]
        m = a.max(axis=1, keepdims=True)
        e = np.exp(a - m)
        z = e.sum(axis=1, keepdims=True)
        O[r] = (e / z) @ Vs
        lse[r] = m[:, 0] + np.log(z[:, 0])
    return O, lse


def sparse_attention(q_bits, k_bits, v_bits, idx, *, scale: Optional[float] = None,
                     pos_offset: int = 0):
    """All rows of all batch entries: O [B, n_q, H, D], lse [B, n_q, H]."""
    qb = np.asarray(q_bits)
    B, n_q, H, D = qb.shape
    O = np.zeros((B, n_q, H, D))
    L = np.zeros((B, n_q, H))
    I = np.asarray(idx)
    for b in range(B):
        O[b], L[b] = sparse_attention_rows(q_bits, k_bits, v_bits, I[b] if I.ndim == 3 else I,
                                           range(n_q), scale=scale, pos_offset=pos_offset,
                                           batch=b)
    return O, L
