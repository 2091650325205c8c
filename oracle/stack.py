"""The IndexCache layer loop (paper, Figure 2: standard DSA runs the indexer at
every layer; IndexCache adds one branch so that F layers compute and cache fresh
indices and S layers reuse the cached ones; the cache is a single index tensor
overwritten at each F layer).

    buf = None
    for l in layers:
        if P[l] == 'F': buf = top-k(indexer_l)      # overwrite the cache
        O_l = sparse_attention_l(buf)               # S layers reuse buf

An S layer therefore uses the indices of the greatest F layer before it.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .attention import sparse_attention_rows
from .indexer import indexer_scores_rows, topk_from_scores
from .pattern import resolve_pattern


def run_stack(layers: List[dict], topk: int, *, pattern: Optional[str] = None, freq: int = 0,
              rows: Optional[Sequence[int]] = None, pos_offset: int = 0, batch: int = 0,
              scale: Optional[float] = None):
    """layers[l] holds host bits: q_idx, k_idx, w, dtype, (q_scale, k_scale), q, k, v.
    Returns (resolved pattern, per-layer idx [R, topk], per-layer O [R, H, D],
    per-layer lse [R, H]) for the chosen rows of one batch entry."""
    P = resolve_pattern(len(layers), pattern, freq)
    n_q = layers[0]["w"].shape[1]
    rows = list(range(n_q)) if rows is None else list(rows)
    buf = None
    idxs, outs, lses = [], [], []
    for l, L in enumerate(layers):
        if P[l] == "F":
            sc = indexer_scores_rows(L["q_idx"], L["k_idx"], L["w"], rows, dtype=L["dtype"],
                                     q_scale=L.get("q_scale"), k_scale=L.get("k_scale"),
                                     pos_offset=pos_offset, batch=batch)
            buf = topk_from_scores(sc, topk, pos_offset=pos_offset, rows=rows)
        # the attention rows are addressed by query row number; buf is [R, topk]
        full_idx = np.full((n_q, topk), -1, dtype=np.int32)
        full_idx[rows] = buf
        O, lse = sparse_attention_rows(L["q"], L["k"], L["v"], full_idx, rows, scale=scale,
                                       pos_offset=pos_offset, batch=batch)
        idxs.append(buf.copy())
        outs.append(O)
        lses.append(lse)
    return P, idxs, outs, lses
