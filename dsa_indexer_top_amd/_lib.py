"""ctypes view of libdsa's C ABI (include/dsa.h). Marshalling only."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_OK = 0
DSA_ERR_INVALID_ARGUMENT = 1
DSA_ERR_UNSUPPORTED = 2
DSA_ERR_BAD_PATTERN = 3
DSA_ERR_WORKSPACE = 4
DSA_ERR_HIP = 5

DSA_STATIC_SCRATCH_BYTES = 64 << 20   # include/dsa.h

DSA_BF16 = 0
DSA_FP8_E4M3FN = 1

# Every symbol include/dsa.h declares.
EXPORTS = (
    "dsa_abi_version",
    "dsa_indexer_workspace_size",
    "dsa_attn_workspace_size",
    "dsa_stack_workspace_size",
    "dsa_resolve_pattern",
    "dsa_indexer_scores_topk",
    "dsa_indexer_scores_topk_static",
    "dsa_sparse_attn",
    "dsa_layer_stack_run",
    "dsa_chunked_stack_workspace_size",
    "dsa_layer_stack_run_chunked",
    "dsa_quantize_fp8_rows",
    "dsa_paged_indexer_topk",
    "dsa_paged_sparse_attn",
    "dsa_paged_layer_stack_run",
    "dsa_paged_append_rows",
    "dsa_topk_overlap",
    "dsa_similarity_pattern",
    "dsa_status_string",
    "dsa_last_error",
)


class IndexerArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_uint32),
        ("B", c_int32), ("n_q", c_int32), ("n_k", c_int32), ("q_pos_offset", c_int32),
        ("n_heads", c_int32), ("head_dim", c_int32), ("topk", c_int32),
        ("dtype", c_int32),
        ("q", c_void_p), ("k", c_void_p), ("w", c_void_p),
        ("q_scale", c_void_p), ("k_scale", c_void_p),
        ("out_idx", c_void_p), ("out_scores", c_void_p), ("debug_full_scores", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("phase_events", c_void_p),
    ]


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_uint32),
        ("B", c_int32), ("n_q", c_int32), ("n_k", c_int32), ("q_pos_offset", c_int32),
        ("n_heads", c_int32), ("head_dim", c_int32), ("topk", c_int32),
        ("scale", c_float),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("idx", c_void_p),
        ("out", c_void_p), ("lse", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("phase_events", c_void_p),
    ]


class PagedKVArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_uint32),
        ("max_seq_len", c_int32), ("page_size", c_int32), ("max_pages", c_int32), ("num_pages", c_int32),
        ("seq_lens", c_void_p), ("block_table", c_void_p),
    ]


class StackArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_uint32),
        ("n_layers", c_int32),
        ("indexer", IndexerArgs),
        ("attn", AttnArgs),
        ("q_idx", c_void_p), ("k_idx", c_void_p), ("w", c_void_p),
        ("q_scale", c_void_p), ("k_scale", c_void_p),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p),
        ("out", c_void_p), ("lse", c_void_p),
        ("idx_buf", c_void_p),
        ("layer_events", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Loads libdsa.so (built in-tree by build.py). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libdsa.so not found at {LIB_PATH}: run __graft_entry__.build() "
                           "(or python dsa_indexer_top_amd/build.py) first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.dsa_abi_version.restype = c_int32
    lib.dsa_abi_version.argtypes = []
    for name, argt in (("dsa_indexer_workspace_size", POINTER(IndexerArgs)),
                       ("dsa_attn_workspace_size", POINTER(AttnArgs)),
                       ("dsa_stack_workspace_size", POINTER(StackArgs))):
        f = getattr(lib, name)
        f.restype = c_int32
        f.argtypes = [argt, POINTER(c_size_t)]
    lib.dsa_resolve_pattern.restype = c_int32
    lib.dsa_resolve_pattern.argtypes = [c_int32, c_char_p, c_int32, ctypes.c_char_p]
    lib.dsa_indexer_scores_topk.restype = c_int32
    lib.dsa_indexer_scores_topk.argtypes = [POINTER(IndexerArgs), c_void_p]
    lib.dsa_indexer_scores_topk_static.restype = c_int32
    lib.dsa_indexer_scores_topk_static.argtypes = [POINTER(IndexerArgs), c_void_p]
    lib.dsa_sparse_attn.restype = c_int32
    lib.dsa_sparse_attn.argtypes = [POINTER(AttnArgs), c_void_p]
    lib.dsa_layer_stack_run.restype = c_int32
    lib.dsa_layer_stack_run.argtypes = [POINTER(StackArgs), c_char_p, c_int32, c_void_p]
    lib.dsa_chunked_stack_workspace_size.restype = c_int32
    lib.dsa_chunked_stack_workspace_size.argtypes = [POINTER(StackArgs), c_int32, POINTER(c_size_t)]
    lib.dsa_layer_stack_run_chunked.restype = c_int32
    lib.dsa_layer_stack_run_chunked.argtypes = [POINTER(StackArgs), c_int32, c_char_p, c_int32, c_void_p]
    lib.dsa_paged_indexer_topk.restype = c_int32
    lib.dsa_paged_indexer_topk.argtypes = [POINTER(IndexerArgs), POINTER(PagedKVArgs), c_void_p]
    lib.dsa_paged_sparse_attn.restype = c_int32
    lib.dsa_paged_sparse_attn.argtypes = [POINTER(AttnArgs), POINTER(PagedKVArgs), c_void_p]
    lib.dsa_paged_layer_stack_run.restype = c_int32
    lib.dsa_paged_layer_stack_run.argtypes = [POINTER(StackArgs), POINTER(PagedKVArgs), c_char_p, c_int32, c_void_p]
    lib.dsa_paged_append_rows.restype = c_int32
    lib.dsa_paged_append_rows.argtypes = [c_void_p, c_int32, c_int32, c_void_p, POINTER(PagedKVArgs), c_void_p]
    lib.dsa_topk_overlap.restype = c_int32
    lib.dsa_topk_overlap.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p]
    lib.dsa_similarity_pattern.restype = c_int32
    lib.dsa_similarity_pattern.argtypes = [c_int32, POINTER(ctypes.c_int64), c_int32, ctypes.c_char_p]
    lib.dsa_quantize_fp8_rows.restype = c_int32
    lib.dsa_quantize_fp8_rows.argtypes = [c_void_p, ctypes.c_int64, c_int32, c_void_p, c_void_p, c_void_p]
    lib.dsa_status_string.restype = c_char_p
    lib.dsa_status_string.argtypes = [c_int32]
    lib.dsa_last_error.restype = c_char_p
    lib.dsa_last_error.argtypes = []
    _lib = lib
    return lib
