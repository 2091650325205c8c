"""dsa_indexer_top_amd - the DeepSeek-Sparse-Attention hot path on MI355X.

The lightning indexer fused with exact per-query top-k, sparse attention over
the selected tokens, and the IndexCache F/S layer stack, as hand-written HIP
kernels for gfx950 behind the C ABI in include/dsa.h (libdsa.so, built in-tree
by build.py). This package is the Python binding of that library.
"""
from ._lib import load as _load_lib, LIB_PATH  # noqa: F401
from .api import (  # noqa: F401
    DsaError,
    IndexerResult,
    LayerStack,
    PagedKV,
    abi_version,
    attn_workspace_size,
    indexer_scores_topk,
    indexer_workspace_size,
    paged_append_rows,
    paged_indexer_topk,
    paged_sparse_attn,
    quantize_fp8_rows,
    similarity_pattern,
    topk_overlap,
    resolve_pattern,
    sparse_attn,
)


def load():
    """Loads libdsa.so; raises RuntimeError if it has not been built."""
    return _load_lib()
