"""Python binding of libdsa: torch tensors in, C ABI calls out.

This layer only marshals arguments (shape/dtype checks, output and workspace
allocation with torch, the current HIP stream); every step of the computation
runs in libdsa's HIP kernels. There is no fallback: if libdsa.so is missing,
every call raises.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

from . import _lib as L


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [status {status}]")
        self.status = status


def load():
    return L.load()


def _check(status: int):
    if status != L.DSA_OK:
        lib = L.load()
        name = lib.dsa_status_string(status).decode()
        msg = lib.dsa_last_error().decode()
        raise DsaError(status, f"{name}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def abi_version() -> int:
    return int(L.load().dsa_abi_version())


def resolve_pattern(n_layers: int, pattern: Optional[str] = None, freq: int = 0) -> str:
    """IndexCache pattern resolution through the library (pure host code)."""
    buf = ctypes.create_string_buffer(max(n_layers, 0) + 1)
    pat = None if pattern is None else pattern.encode()
    _check(L.load().dsa_resolve_pattern(int(n_layers), pat, int(freq), buf))
    return buf.value.decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.DSA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return L.DSA_FP8_E4M3FN
    raise TypeError(f"indexer inputs must be bfloat16 or float8_e4m3fn, got {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, shape=None):
    """Type, dtype, rank, exact shape and contiguity of a caller tensor. The C
    ABI carries no shapes, so every tensor a kernel reads or writes is checked
    here; devices are checked afterwards by _on_gpu (shape errors first, so
    they are reported the same way on a host without a GPU)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(*named):
    """Every given (name, tensor) pair (None tensors skipped) is a GPU tensor,
    all on one device; returns that device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev


def _opt_out(spec, name: str, dtype, shape):
    """An optional output argument: True (allocate later), False/None (absent)
    or a caller tensor, which must have exactly this dtype and shape."""
    if spec is True or spec is False or spec is None:
        return spec
    _need(spec, name, dtype=dtype, shape=shape)
    return spec


def indexer_args(B, n_q, n_k, pos_offset, H, D, topk, dtype_code) -> L.IndexerArgs:
    a = L.IndexerArgs()
    a.struct_size = ctypes.sizeof(L.IndexerArgs)
    a.B, a.n_q, a.n_k, a.q_pos_offset = B, n_q, n_k, pos_offset
    a.n_heads, a.head_dim, a.topk, a.dtype = H, D, topk, dtype_code
    return a


def attn_args(B, n_q, n_k, pos_offset, H, D, topk, scale) -> L.AttnArgs:
    a = L.AttnArgs()
    a.struct_size = ctypes.sizeof(L.AttnArgs)
    a.B, a.n_q, a.n_k, a.q_pos_offset = B, n_q, n_k, pos_offset
    a.n_heads, a.head_dim, a.topk, a.scale = H, D, topk, float(scale)
    return a


def indexer_workspace_size(B, n_q, n_k, H, D, topk, dtype_code=L.DSA_BF16, pos_offset=None) -> int:
    if pos_offset is None:
        pos_offset = n_k - n_q
    a = indexer_args(B, n_q, n_k, pos_offset, H, D, topk, dtype_code)
    n = ctypes.c_size_t(0)
    _check(L.load().dsa_indexer_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return int(n.value)


def attn_workspace_size(B, n_q, n_k, H, D, topk, pos_offset=None) -> int:
    if pos_offset is None:
        pos_offset = n_k - n_q
    a = attn_args(B, n_q, n_k, pos_offset, H, D, topk, 0.0)
    n = ctypes.c_size_t(0)
    _check(L.load().dsa_attn_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return int(n.value)


def _workspace(nbytes: int, device, given: Optional[torch.Tensor]):
    if given is not None:
        _need(given, "workspace")
        _on_gpu(("workspace", given))
        if given.device != device:
            raise ValueError(f"workspace is on {given.device}, the other tensors on {device}")
        if given.numel() * given.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return given
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class IndexerResult:
    idx: torch.Tensor                    # [B, n_q, topk] int32
    scores: Optional[torch.Tensor]       # [B, n_q, topk] fp32
    full_scores: Optional[torch.Tensor]  # [B, n_q, n_k] fp32 (test mode)


def indexer_scores_topk(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, topk: int, *,
                        q_scale: Optional[torch.Tensor] = None,
                        k_scale: Optional[torch.Tensor] = None,
                        pos_offset: Optional[int] = None,
                        out_idx: Optional[torch.Tensor] = None,
                        out_scores=False, debug_full_scores=False,
                        workspace: Optional[torch.Tensor] = None,
                        stream=None, phase_events=None, static_scratch: bool = False) -> IndexerResult:
    """Lightning-indexer scores + exact per-query top-k (dsa_indexer_scores_topk).

    static_scratch=True calls dsa_indexer_scores_topk_static instead: no
    workspace is allocated or passed (the library's static device scratch is
    used; pass out_idx and the other outputs to allocate nothing at all).

    q [B, n_q, H, D], k [B, n_k, D] (bf16 or float8_e4m3fn), w [B, n_q, H] fp32,
    fp8: q_scale [B, n_q], k_scale [B, n_k] fp32. out_scores / debug_full_scores
    may be True (allocate), a tensor, or False. debug_full_scores is pre-filled
    with NaN so that the entries the kernel does not write stay recognisable."""
    _need(q, "q", ndim=4)
    B, n_q, H, D = q.shape
    _need(k, "k", dtype=q.dtype, ndim=3)
    n_k = k.shape[1]
    _need(k, "k", shape=(B, n_k, D))
    _need(w, "w", dtype=torch.float32, shape=(B, n_q, H))
    code = _dtype_code(q)
    if code == L.DSA_FP8_E4M3FN:
        _need(q_scale, "q_scale", dtype=torch.float32, shape=(B, n_q))
        _need(k_scale, "k_scale", dtype=torch.float32, shape=(B, n_k))
    elif q_scale is not None or k_scale is not None:
        raise ValueError("q_scale and k_scale are for fp8 inputs only")
    if pos_offset is None:
        pos_offset = n_k - n_q
    if out_idx is not None:
        _need(out_idx, "out_idx", dtype=torch.int32, shape=(B, n_q, topk))
    out_scores = _opt_out(out_scores, "out_scores", torch.float32, (B, n_q, topk))
    debug_full_scores = _opt_out(debug_full_scores, "debug_full_scores", torch.float32, (B, n_q, n_k))
    dev = _on_gpu(("q", q), ("k", k), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale), ("out_idx", out_idx),
                  ("out_scores", out_scores if isinstance(out_scores, torch.Tensor) else None),
                  ("debug_full_scores", debug_full_scores if isinstance(debug_full_scores, torch.Tensor) else None))
    if out_idx is None:
        out_idx = torch.empty((B, n_q, topk), dtype=torch.int32, device=dev)
    sc = None
    if out_scores is True:
        sc = torch.empty((B, n_q, topk), dtype=torch.float32, device=dev)
    elif isinstance(out_scores, torch.Tensor):
        sc = out_scores
    full = None
    if debug_full_scores is True:
        full = torch.full((B, n_q, n_k), float("nan"), dtype=torch.float32, device=dev)
    elif isinstance(debug_full_scores, torch.Tensor):
        full = debug_full_scores
    a = indexer_args(B, n_q, n_k, pos_offset, H, D, topk, code)
    if static_scratch:
        if workspace is not None:
            raise ValueError("static_scratch takes no workspace")
        ws = None
    else:
        nbytes = ctypes.c_size_t(0)
        _check(L.load().dsa_indexer_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
        ws = _workspace(int(nbytes.value), dev, workspace)
    a.q, a.k, a.w = _ptr(q), _ptr(k), _ptr(w)
    a.q_scale, a.k_scale = _ptr(q_scale), _ptr(k_scale)
    a.out_idx, a.out_scores, a.debug_full_scores = _ptr(out_idx), _ptr(sc), _ptr(full)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    keep = _event_array(phase_events, 3)
    a.phase_events = None if keep is None else ctypes.cast(keep, ctypes.c_void_p)
    fn = L.load().dsa_indexer_scores_topk_static if static_scratch else L.load().dsa_indexer_scores_topk
    _check(fn(ctypes.byref(a), _stream(stream)))
    return IndexerResult(out_idx, sc, full)


def sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, *,
                scale: float = 0.0, pos_offset: Optional[int] = None,
                out: Optional[torch.Tensor] = None, lse=False,
                workspace: Optional[torch.Tensor] = None, stream=None, phase_events=None):
    """Sparse attention (dsa_sparse_attn): q [B, n_q, H, D], k/v [B, n_k, D] bf16,
    idx [B, n_q, topk] int32. Returns (out bf16 [B, n_q, H, D], lse or None)."""
    _need(q, "q", dtype=torch.bfloat16, ndim=4)
    B, n_q, H, D = q.shape
    _need(k, "k", dtype=torch.bfloat16, ndim=3)
    n_k = k.shape[1]
    _need(k, "k", shape=(B, n_k, D))
    _need(v, "v", dtype=torch.bfloat16, shape=(B, n_k, D))
    _need(idx, "idx", dtype=torch.int32, ndim=3)
    topk = idx.shape[2]
    _need(idx, "idx", shape=(B, n_q, topk))
    if pos_offset is None:
        pos_offset = n_k - n_q
    if out is not None:
        _need(out, "out", dtype=torch.bfloat16, shape=(B, n_q, H, D))
    lse = _opt_out(lse, "lse", torch.float32, (B, n_q, H))
    dev = _on_gpu(("q", q), ("k", k), ("v", v), ("idx", idx), ("out", out),
                  ("lse", lse if isinstance(lse, torch.Tensor) else None))
    if out is None:
        out = torch.empty((B, n_q, H, D), dtype=torch.bfloat16, device=dev)
    lse_t = None
    if lse is True:
        lse_t = torch.empty((B, n_q, H), dtype=torch.float32, device=dev)
    elif isinstance(lse, torch.Tensor):
        lse_t = lse
    a = attn_args(B, n_q, n_k, pos_offset, H, D, topk, scale)
    nbytes = ctypes.c_size_t(0)
    _check(L.load().dsa_attn_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws = _workspace(int(nbytes.value), dev, workspace)
    a.q, a.k, a.v, a.idx, a.out, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out), _ptr(lse_t)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    keep = _event_array(phase_events, 2)
    a.phase_events = None if keep is None else ctypes.cast(keep, ctypes.c_void_p)
    _check(L.load().dsa_sparse_attn(ctypes.byref(a), _stream(stream)))
    return out, lse_t


class PagedKV:
    """Layout of a paged, ragged decode cache (dsa_paged_kv): request b has
    seq_lens[b] tokens and token s sits in page block_table[b, s // page_size],
    slot s % page_size, of each page pool ([num_pages, page_size, ...]).
    seq_lens [B] and block_table [B, max_pages] are int32 GPU tensors;
    max_seq_len is a host upper bound of seq_lens."""

    def __init__(self, seq_lens: torch.Tensor, block_table: torch.Tensor, page_size: int, num_pages: int,
                 max_seq_len: int):
        _need(seq_lens, "seq_lens", dtype=torch.int32, ndim=1)
        _need(block_table, "block_table", dtype=torch.int32, ndim=2)
        if block_table.shape[0] != seq_lens.shape[0]:
            raise ValueError("block_table must be [B, max_pages]")
        self.device = _on_gpu(("seq_lens", seq_lens), ("block_table", block_table))
        self.seq_lens, self.block_table = seq_lens, block_table
        self.page_size, self.num_pages, self.max_seq_len = int(page_size), int(num_pages), int(max_seq_len)
        self.B, self.max_pages = block_table.shape
        a = L.PagedKVArgs()
        a.struct_size = ctypes.sizeof(L.PagedKVArgs)
        a.max_seq_len, a.page_size = self.max_seq_len, self.page_size
        a.max_pages, a.num_pages = self.max_pages, self.num_pages
        a.seq_lens, a.block_table = _ptr(seq_lens), _ptr(block_table)
        self.args = a

    def check_pool(self, pool: torch.Tensor, name: str, row_shape, dtype=None):
        _need(pool, name, dtype=dtype)
        if tuple(pool.shape) != (self.num_pages, self.page_size, *row_shape):
            raise ValueError(f"{name} must be [num_pages, page_size, {', '.join(map(str, row_shape))}]")
        _on_gpu((name, pool))
        if pool.device != self.device:
            raise ValueError(f"{name} is on {pool.device}, the cache layout on {self.device}")


def paged_indexer_topk(q: torch.Tensor, k_pool: torch.Tensor, w: torch.Tensor, topk: int, kv: PagedKV, *,
                       q_scale: Optional[torch.Tensor] = None, k_scale_pool: Optional[torch.Tensor] = None,
                       out_idx: Optional[torch.Tensor] = None, out_scores=False, debug_full_scores=False,
                       workspace: Optional[torch.Tensor] = None, stream=None,
                       phase_events=None) -> IndexerResult:
    """Decode indexer + top-k over a paged cache (dsa_paged_indexer_topk).
    q [B, 1, H, D], w [B, 1, H], k_pool [num_pages, page_size, D] (bf16 or
    float8_e4m3fn); fp8: q_scale [B, 1], k_scale_pool [num_pages, page_size].
    Indices are logical token positions; debug_full_scores is [B, 1, max_seq_len]."""
    _need(q, "q", ndim=4)
    B, n_q, H, D = q.shape
    if n_q != 1 or B != kv.B:
        raise ValueError("q must be [B, 1, H, D] with B = kv.B")
    kv.check_pool(k_pool, "k_pool", (D,), dtype=q.dtype)
    _need(w, "w", dtype=torch.float32, shape=(B, 1, H))
    code = _dtype_code(q)
    if code == L.DSA_FP8_E4M3FN:
        _need(q_scale, "q_scale", dtype=torch.float32, shape=(B, 1))
        kv.check_pool(k_scale_pool, "k_scale_pool", (), dtype=torch.float32)
    elif q_scale is not None or k_scale_pool is not None:
        raise ValueError("q_scale and k_scale_pool are for fp8 inputs only")
    n_k = kv.max_seq_len
    if out_idx is not None:
        _need(out_idx, "out_idx", dtype=torch.int32, shape=(B, 1, topk))
    out_scores = _opt_out(out_scores, "out_scores", torch.float32, (B, 1, topk))
    debug_full_scores = _opt_out(debug_full_scores, "debug_full_scores", torch.float32, (B, 1, n_k))
    dev = _on_gpu(("q", q), ("w", w), ("q_scale", q_scale), ("out_idx", out_idx),
                  ("out_scores", out_scores if isinstance(out_scores, torch.Tensor) else None),
                  ("debug_full_scores", debug_full_scores if isinstance(debug_full_scores, torch.Tensor) else None))
    if dev != kv.device:
        raise ValueError(f"q is on {dev}, the cache layout on {kv.device}")
    if out_idx is None:
        out_idx = torch.empty((B, 1, topk), dtype=torch.int32, device=dev)
    sc = torch.empty((B, 1, topk), dtype=torch.float32, device=dev) if out_scores is True else (
        out_scores if isinstance(out_scores, torch.Tensor) else None)
    full = torch.full((B, 1, n_k), float("nan"), dtype=torch.float32, device=dev) if debug_full_scores is True \
        else (debug_full_scores if isinstance(debug_full_scores, torch.Tensor) else None)
    a = indexer_args(B, 1, n_k, n_k - 1, H, D, topk, code)
    nbytes = ctypes.c_size_t(0)
    _check(L.load().dsa_indexer_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws = _workspace(int(nbytes.value), dev, workspace)
    a.q, a.k, a.w = _ptr(q), _ptr(k_pool), _ptr(w)
    a.q_scale, a.k_scale = _ptr(q_scale), _ptr(k_scale_pool)
    a.out_idx, a.out_scores, a.debug_full_scores = _ptr(out_idx), _ptr(sc), _ptr(full)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    keep = _event_array(phase_events, 3)
    a.phase_events = None if keep is None else ctypes.cast(keep, ctypes.c_void_p)
    _check(L.load().dsa_paged_indexer_topk(ctypes.byref(a), ctypes.byref(kv.args), _stream(stream)))
    return IndexerResult(out_idx, sc, full)


def paged_sparse_attn(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, idx: torch.Tensor,
                      kv: PagedKV, *, scale: float = 0.0, out: Optional[torch.Tensor] = None, lse=False,
                      workspace: Optional[torch.Tensor] = None, stream=None, phase_events=None):
    """Decode sparse attention over a paged cache (dsa_paged_sparse_attn): q
    [B, 1, H, D], k_pool / v_pool [num_pages, page_size, D] bf16, idx [B, 1, topk]
    logical positions. Returns (out [B, 1, H, D] bf16, lse or None)."""
    _need(q, "q", dtype=torch.bfloat16, ndim=4)
    B, n_q, H, D = q.shape
    if n_q != 1 or B != kv.B:
        raise ValueError("q must be [B, 1, H, D] with B = kv.B")
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        kv.check_pool(t, nm, (D,), dtype=torch.bfloat16)
    _need(idx, "idx", dtype=torch.int32, ndim=3)
    topk = idx.shape[2]
    _need(idx, "idx", shape=(B, 1, topk))
    if out is not None:
        _need(out, "out", dtype=torch.bfloat16, shape=(B, 1, H, D))
    lse = _opt_out(lse, "lse", torch.float32, (B, 1, H))
    dev = _on_gpu(("q", q), ("idx", idx), ("out", out), ("lse", lse if isinstance(lse, torch.Tensor) else None))
    if dev != kv.device:
        raise ValueError(f"q is on {dev}, the cache layout on {kv.device}")
    n_k = kv.max_seq_len
    if out is None:
        out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=dev)
    lse_t = torch.empty((B, 1, H), dtype=torch.float32, device=dev) if lse is True else (
        lse if isinstance(lse, torch.Tensor) else None)
    a = attn_args(B, 1, n_k, n_k - 1, H, D, topk, scale)
    nbytes = ctypes.c_size_t(0)
    _check(L.load().dsa_attn_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws = _workspace(int(nbytes.value), dev, workspace)
    a.q, a.k, a.v, a.idx, a.out, a.lse = _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(idx), _ptr(out), _ptr(lse_t)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    keep = _event_array(phase_events, 2)
    a.phase_events = None if keep is None else ctypes.cast(keep, ctypes.c_void_p)
    _check(L.load().dsa_paged_sparse_attn(ctypes.byref(a), ctypes.byref(kv.args), _stream(stream)))
    return out, lse_t


def paged_append_rows(src: torch.Tensor, pool: torch.Tensor, kv: PagedKV, stream=None):
    """dsa_paged_append_rows: src [B, ...] (one row per request) goes to each
    request's last position, seq_lens[b] - 1, of pool [num_pages, page_size, ...]."""
    _need(src, "src")
    B = src.shape[0]
    if B != kv.B:
        raise ValueError("src must have one row per request")
    kv.check_pool(pool, "pool", tuple(src.shape[1:]), dtype=src.dtype)
    _on_gpu(("src", src), ("pool", pool))
    if src.device != kv.device:
        raise ValueError(f"src is on {src.device}, the cache layout on {kv.device}")
    row_bytes = (src.numel() // B) * src.element_size()
    _check(L.load().dsa_paged_append_rows(_ptr(src), B, row_bytes, _ptr(pool), ctypes.byref(kv.args),
                                          _stream(stream)))


def topk_overlap(idx: torch.Tensor, n_k: int, *, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dsa_topk_overlap: idx [n_layers, rows, topk] int32 (GPU) -> inter
    [n_layers, n_layers] int64 (GPU), inter[a][b] = sum over rows of the number
    of tokens both layers selected. The overlap ratio is inter[a][b] / inter[a][a]."""
    _need(idx, "idx", dtype=torch.int32, ndim=3)
    n_layers, rows, topk = idx.shape
    if out is not None:
        _need(out, "out", dtype=torch.int64, shape=(n_layers, n_layers))
    dev = _on_gpu(("idx", idx), ("out", out))
    if out is None:
        out = torch.empty((n_layers, n_layers), dtype=torch.int64, device=dev)
    _check(L.load().dsa_topk_overlap(_ptr(idx), n_layers, rows, topk, int(n_k), _ptr(out), _stream(stream)))
    return out


def similarity_pattern(inter, n_full: int) -> str:
    """dsa_similarity_pattern (host): the F/S string with n_full F layers that
    maximises the selections every S layer shares with the last F layer before
    it. inter: [n_layers, n_layers] int64 (torch tensor on any device, or array)."""
    if isinstance(inter, torch.Tensor):
        inter = inter.detach().to("cpu", torch.int64).contiguous()
    else:
        inter = torch.as_tensor(inter, dtype=torch.int64).contiguous()
    n = inter.shape[0]
    if inter.dim() != 2 or inter.shape[1] != n:
        raise ValueError("inter must be square")
    buf = ctypes.create_string_buffer(n + 1)
    ptr = ctypes.cast(inter.data_ptr(), ctypes.POINTER(ctypes.c_int64))
    _check(L.load().dsa_similarity_pattern(n, ptr, int(n_full), buf))
    return buf.value.decode()


def quantize_fp8_rows(x: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                      scale: Optional[torch.Tensor] = None, stream=None):
    """Per-token fp8 quantisation (dsa_quantize_fp8_rows): x is bf16 with the
    token's values in its last dims, given as [..., cols] (q_idx [B, n_q, H, D]
    -> pass x.view(B, n_q, H * D); k_idx [B, n_k, D] as is). Returns (codes as
    float8_e4m3fn with x's shape, scale fp32 with x's shape minus the last dim)."""
    _need(x, "x", dtype=torch.bfloat16)
    if x.dim() < 1:
        raise ValueError("x must have at least one dim")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if out is not None:
        _need(out, "out", dtype=torch.float8_e4m3fn, shape=x.shape)
    if scale is not None:
        _need(scale, "scale", dtype=torch.float32)
        if scale.numel() != rows:
            raise ValueError(f"scale must have one entry per row ({rows}), got {scale.numel()}")
    dev = _on_gpu(("x", x), ("out", out), ("scale", scale))
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev)
    if scale is None:
        scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    _check(L.load().dsa_quantize_fp8_rows(_ptr(x), rows, cols, _ptr(out), _ptr(scale), _stream(stream)))
    return out, scale


def _event_array(events, n):
    """Host array of hipEvent_t handles from torch.cuda.Event objects (or None)."""
    if events is None:
        return None
    if len(events) != n:
        raise ValueError(f"phase_events needs {n} events")
    arr = (ctypes.c_void_p * n)()
    for i, e in enumerate(events):
        if e.cuda_event == 0:   # torch creates the underlying event lazily
            e.record()
        arr[i] = e.cuda_event
    return arr


def _ptr_array(ts: Sequence[Optional[torch.Tensor]]):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if t is None else t.data_ptr()
    return arr


class LayerStack:
    """A prepared dsa_layer_stack_run call: per-layer tensors, the shared index
    buffer (IndexCache's cache) and one workspace, reusable across runs."""

    def __init__(self, layers: List[dict], topk: int, *, scale: float = 0.0,
                 pos_offset: Optional[int] = None, lse: bool = False, shared_out: bool = False,
                 events: bool = False, kv: Optional[PagedKV] = None, chunk_rows: Optional[int] = None):
        """kv: a PagedKV for one decode step over paged caches (every layer's
        k_idx, k_scale, k and v are then page pools and n_q must be 1).
        chunk_rows: prefill the rows in chunks of this many (one sequence,
        B = 1; dsa_layer_stack_run_chunked): the index buffer then holds one
        chunk's rows and the workspace is sized for one chunk."""
        if not layers:
            raise ValueError("layers is empty")
        l0 = layers[0]
        _need(l0["q_idx"], "layers[0].q_idx", ndim=4)
        _need(l0["q"], "layers[0].q", dtype=torch.bfloat16, ndim=4)
        B, n_q, H_I, D_I = l0["q_idx"].shape
        _, _, H, D = l0["q"].shape
        code = _dtype_code(l0["q_idx"])
        fp8 = code == L.DSA_FP8_E4M3FN
        if kv is None:
            _need(l0["k_idx"], "layers[0].k_idx", ndim=3)
            n_k = l0["k_idx"].shape[1]
        else:
            n_k = kv.max_seq_len
            if n_q != 1:
                raise ValueError("a paged stack is one decode step: n_q must be 1")
        if chunk_rows is not None and (kv is not None or B != 1 or int(chunk_rows) < 1 or events):
            raise ValueError("chunk_rows needs one flat-cache sequence (B = 1), chunk_rows >= 1 and no "
                             "per-layer events")
        named = []
        for i, ly in enumerate(layers):
            pre = f"layers[{i}]."
            _need(ly["q_idx"], pre + "q_idx", dtype=l0["q_idx"].dtype, shape=(B, n_q, H_I, D_I))
            _need(ly["w"], pre + "w", dtype=torch.float32, shape=(B, n_q, H_I))
            _need(ly["q"], pre + "q", dtype=torch.bfloat16, shape=(B, n_q, H, D))
            if kv is None:
                _need(ly["k_idx"], pre + "k_idx", dtype=l0["q_idx"].dtype, shape=(B, n_k, D_I))
                _need(ly["k"], pre + "k", dtype=torch.bfloat16, shape=(B, n_k, D))
                _need(ly["v"], pre + "v", dtype=torch.bfloat16, shape=(B, n_k, D))
            else:
                kv.check_pool(ly["k_idx"], pre + "k_idx", (D_I,), dtype=l0["q_idx"].dtype)
                kv.check_pool(ly["k"], pre + "k", (D,), dtype=torch.bfloat16)
                kv.check_pool(ly["v"], pre + "v", (D,), dtype=torch.bfloat16)
            if fp8:
                _need(ly.get("q_scale"), pre + "q_scale", dtype=torch.float32, shape=(B, n_q))
                if kv is None:
                    _need(ly.get("k_scale"), pre + "k_scale", dtype=torch.float32, shape=(B, n_k))
                else:
                    kv.check_pool(ly.get("k_scale"), pre + "k_scale", (), dtype=torch.float32)
            elif ly.get("q_scale") is not None or ly.get("k_scale") is not None:
                raise ValueError(f"layer {i}: q_scale/k_scale are for fp8 inputs only")
            named += [(pre + nm, ly.get(nm)) for nm in ("q_idx", "k_idx", "w", "q_scale", "k_scale", "q", "k", "v")]
        dev = _on_gpu(*named)
        if kv is not None and dev != kv.device:
            raise ValueError(f"the layers are on {dev}, the cache layout on {kv.device}")
        self.kv = kv
        self.chunk_rows = None if chunk_rows is None else int(chunk_rows)
        if pos_offset is None:
            pos_offset = n_k - n_q
        self.layers = layers
        buf_rows = n_q if self.chunk_rows is None else min(self.chunk_rows, n_q)
        self.idx_buf = torch.empty((B, buf_rows, topk), dtype=torch.int32, device=dev)
        if shared_out:
            o = torch.empty((B, n_q, H, D), dtype=torch.bfloat16, device=dev)
            self.outs = [o] * len(layers)
        else:
            self.outs = [torch.empty((B, n_q, H, D), dtype=torch.bfloat16, device=dev) for _ in layers]
        self.lses = ([torch.empty((B, n_q, H), dtype=torch.float32, device=dev) for _ in layers]
                     if lse else None)
        a = L.StackArgs()
        a.struct_size = ctypes.sizeof(L.StackArgs)
        a.n_layers = len(layers)
        a.indexer = indexer_args(B, n_q, n_k, pos_offset, H_I, D_I, topk, code)
        a.attn = attn_args(B, n_q, n_k, pos_offset, H, D, topk, scale)
        self._keep = [
            _ptr_array([ly["q_idx"] for ly in layers]), _ptr_array([ly["k_idx"] for ly in layers]),
            _ptr_array([ly["w"] for ly in layers]),
            _ptr_array([ly["q_scale"] for ly in layers]) if fp8 else None,
            _ptr_array([ly["k_scale"] for ly in layers]) if fp8 else None,
            _ptr_array([ly["q"] for ly in layers]), _ptr_array([ly["k"] for ly in layers]),
            _ptr_array([ly["v"] for ly in layers]), _ptr_array(self.outs),
            _ptr_array(self.lses) if self.lses is not None else None,
        ]
        names = ["q_idx", "k_idx", "w", "q_scale", "k_scale", "q", "k", "v", "out", "lse"]
        for nm, arr in zip(names, self._keep):
            setattr(a, nm, None if arr is None else ctypes.cast(arr, ctypes.c_void_p))
        a.idx_buf = _ptr(self.idx_buf)
        self.events = None
        if events:
            self.events = [torch.cuda.Event(enable_timing=True) for _ in range(len(layers) + 1)]
            ev = _event_array(self.events, len(self.events))
            self._keep.append(ev)
            a.layer_events = ctypes.cast(ev, ctypes.c_void_p)
        n = ctypes.c_size_t(0)
        if self.chunk_rows is None:
            _check(L.load().dsa_stack_workspace_size(ctypes.byref(a), ctypes.byref(n)))
        else:
            _check(L.load().dsa_chunked_stack_workspace_size(ctypes.byref(a), self.chunk_rows, ctypes.byref(n)))
        self.workspace = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)
        a.workspace = _ptr(self.workspace)
        a.workspace_bytes = self.workspace.numel()
        self.args = a

    def run(self, pattern: Optional[str] = None, freq: int = 0, stream=None):
        pat = None if pattern is None else pattern.encode()
        if self.chunk_rows is not None:
            _check(L.load().dsa_layer_stack_run_chunked(ctypes.byref(self.args), self.chunk_rows, pat, int(freq),
                                                        _stream(stream)))
        elif self.kv is None:
            _check(L.load().dsa_layer_stack_run(ctypes.byref(self.args), pat, int(freq), _stream(stream)))
        else:
            _check(L.load().dsa_paged_layer_stack_run(ctypes.byref(self.args), ctypes.byref(self.kv.args), pat,
                                                      int(freq), _stream(stream)))
        return self.idx_buf, self.outs, self.lses

    def layer_times_ms(self) -> List[float]:
        """Per-layer durations from the recorded layer events (after a sync)."""
        if not self.events:
            raise RuntimeError("created without events=True")
        return [self.events[i].elapsed_time(self.events[i + 1]) for i in range(len(self.events) - 1)]
