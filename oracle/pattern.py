"""IndexCache layer pattern: which layers keep (F) or reuse (S) the indexer.

IndexCache repository README, "Step 3: Launch with IndexCache":
  * Option A, uniform interleaving: with index_topk_freq = N, every N-th layer
    keeps its indexer (N = 2 removes half of the indexers). Read here as layer
    l is Full iff l % N == 0, so layer 0 always runs its indexer.
  * Option B, custom pattern: one character per DSA layer, 'F' runs the
    indexer, 'S' reuses the cached indices.
  * Default behavior: with neither option set, every layer runs its indexer
    (plain DSA).
The two options are alternatives; setting both is rejected. A pattern must
start with 'F' because an S layer reuses indices that an earlier F layer
cached (paper, Figure 2 caption: the cache holds the indices of the most
recent F layer).
"""
from __future__ import annotations

from typing import Optional


class PatternError(ValueError):
    pass


def resolve_pattern(n_layers: int, pattern: Optional[str] = None, freq: int = 0) -> str:
    """Returns the resolved 'F'/'S' string of length n_layers."""
    if n_layers < 1:
        raise PatternError("n_layers must be >= 1")
    if freq < 0:
        raise PatternError("index_topk_freq must be >= 0")
    if pattern is not None and freq > 0:
        raise PatternError("index_topk_pattern and index_topk_freq are alternatives")
    if pattern is not None:
        if len(pattern) != n_layers:
            raise PatternError("pattern length must equal the number of layers")
        if any(c not in "FS" for c in pattern):
            raise PatternError("pattern characters must be 'F' or 'S'")
        if pattern[0] != "F":
            raise PatternError("the first layer must be 'F'")
        return pattern
    if freq > 0:
        return "".join("F" if l % freq == 0 else "S" for l in range(n_layers))
    return "F" * n_layers
