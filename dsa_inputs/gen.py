"""Seeded input generators (draws and dtype casts only; no method arithmetic)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

TENSOR_IDS = {
    "q_idx": 1,
    "k_idx": 2,
    "w": 3,
    "q": 4,
    "k": 5,
    "v": 6,
    "q_scale": 7,
    "k_scale": 8,
    "pattern": 9,
}


def seed_for(config: int, layer: int, tensor: str) -> int:
    """Seed of one tensor of one layer of one workload configuration."""
    return 1_000_000 * int(config) + 1000 * int(layer) + TENSOR_IDS[tensor]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, seed: int, device="cpu") -> torch.Tensor:
    """Standard normal fp32 draw from its own seeded generator."""
    return torch.randn(tuple(shape), generator=_gen(seed, device), device=device,
                       dtype=torch.float32)


def rand_uniform(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    u = torch.rand(tuple(shape), generator=_gen(seed, device), device=device,
                   dtype=torch.float32)
    return u * (hi - lo) + lo


def randint(shape, lo: int, hi_inclusive: int, seed: int, device="cpu") -> torch.Tensor:
    return torch.randint(lo, hi_inclusive + 1, tuple(shape), generator=_gen(seed, device),
                         device=device, dtype=torch.int64)


def to_e4m3_clipped(x: torch.Tensor, clip: float = 8.0) -> torch.Tensor:
    """Round-to-nearest-even cast of clip(x, +-clip) to OCP fp8 e4m3fn."""
    return x.clamp(-clip, clip).to(torch.float8_e4m3fn)


@dataclass
class IndexerInputs:
    """Inputs of one indexer call. Layouts are row-major, last dim contiguous.

    q: [B, n_q, H, D] bf16 or float8_e4m3fn; k: [B, n_k, D] same dtype;
    w: [B, n_q, H] fp32; q_scale: [B, n_q] fp32 and k_scale: [B, n_k] fp32
    (fp8 only, else None). Query t sits at position pos_offset + t.
    """
    q: torch.Tensor
    k: torch.Tensor
    w: torch.Tensor
    q_scale: Optional[torch.Tensor]
    k_scale: Optional[torch.Tensor]
    dtype: str
    pos_offset: int

    @property
    def shape(self):
        B, n_q, H, D = self.q.shape
        return B, n_q, self.k.shape[1], H, D

    def to(self, device) -> "IndexerInputs":
        mv = (lambda t: None if t is None else t.to(device))
        return IndexerInputs(mv(self.q), mv(self.k), mv(self.w), mv(self.q_scale),
                             mv(self.k_scale), self.dtype, self.pos_offset)


@dataclass
class AttnInputs:
    """Sparse-attention inputs: q [B, n_q, H, D], k/v [B, n_k, D], all bf16
    (one KV head shared by the H query heads)."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    pos_offset: int

    def to(self, device) -> "AttnInputs":
        return AttnInputs(self.q.to(device), self.k.to(device), self.v.to(device),
                          self.pos_offset)


def make_indexer_inputs(B: int, n_q: int, n_k: int, H: int, D: int, *, config: int = 0,
                        layer: int = 0, dtype: str = "bf16", w_std: Optional[float] = None,
                        pos_offset: Optional[int] = None, device="cpu") -> IndexerInputs:
    """q_idx, k_idx ~ N(0,1) (bf16, or e4m3 of the draw clipped to +-8 with
    per-token scales ~ U[0.5, 2)); w ~ N(0,1) * w_std, w_std = 1/sqrt(H) unless
    given. pos_offset defaults to n_k - n_q (the queries are the last n_q tokens)."""
    if pos_offset is None:
        pos_offset = n_k - n_q
    qf = randn((B, n_q, H, D), seed_for(config, layer, "q_idx"), device)
    kf = randn((B, n_k, D), seed_for(config, layer, "k_idx"), device)
    w = randn((B, n_q, H), seed_for(config, layer, "w"), device)
    w = w * (w_std if w_std is not None else 1.0 / float(np.sqrt(H)))
    if dtype == "bf16":
        return IndexerInputs(qf.to(torch.bfloat16), kf.to(torch.bfloat16), w.contiguous(),
                             None, None, "bf16", pos_offset)
    if dtype == "fp8":
        qs = rand_uniform((B, n_q), 0.5, 2.0, seed_for(config, layer, "q_scale"), device)
        ks = rand_uniform((B, n_k), 0.5, 2.0, seed_for(config, layer, "k_scale"), device)
        return IndexerInputs(to_e4m3_clipped(qf), to_e4m3_clipped(kf), w.contiguous(), qs, ks,
                             "fp8", pos_offset)
    raise ValueError(f"unknown dtype {dtype}")


def make_int_indexer_inputs(B: int, n_q: int, n_k: int, H: int, D: int, *, seed: int = 7,
                            dtype: str = "bf16", pos_offset: Optional[int] = None,
                            qk_range: int = 3, device="cpu") -> IndexerInputs:
    """Exact-arithmetic inputs: q, k integers in [-qk_range, qk_range] (exact in
    bf16 and e4m3), w in {+-0.5, +-1, +-2}; fp8 scales in {0.5, 1, 2}. Every
    partial sum is then an exact small dyadic number, so fp32 accumulation in any
    order is exact and scores tie often."""
    if pos_offset is None:
        pos_offset = n_k - n_q
    q = randint((B, n_q, H, D), -qk_range, qk_range, seed * 10 + 1, device).float()
    k = randint((B, n_k, D), -qk_range, qk_range, seed * 10 + 2, device).float()
    wv = torch.tensor([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], device=device)
    w = wv[randint((B, n_q, H), 0, 5, seed * 10 + 3, device)].contiguous()
    if dtype == "bf16":
        return IndexerInputs(q.to(torch.bfloat16), k.to(torch.bfloat16), w, None, None,
                             "bf16", pos_offset)
    sv = torch.tensor([0.5, 1.0, 2.0], device=device)
    qs = sv[randint((B, n_q), 0, 2, seed * 10 + 4, device)].contiguous()
    ks = sv[randint((B, n_k), 0, 2, seed * 10 + 5, device)].contiguous()
    return IndexerInputs(q.to(torch.float8_e4m3fn), k.to(torch.float8_e4m3fn), w, qs, ks,
                         "fp8", pos_offset)


def make_attn_inputs(B: int, n_q: int, n_k: int, H: int, D: int, *, config: int = 0,
                     layer: int = 0, pos_offset: Optional[int] = None,
                     device="cpu") -> AttnInputs:
    """q, k, v ~ N(0,1) in bf16; one KV head shared by H query heads."""
    if pos_offset is None:
        pos_offset = n_k - n_q
    q = randn((B, n_q, H, D), seed_for(config, layer, "q"), device).to(torch.bfloat16)
    k = randn((B, n_k, D), seed_for(config, layer, "k"), device).to(torch.bfloat16)
    v = randn((B, n_k, D), seed_for(config, layer, "v"), device).to(torch.bfloat16)
    return AttnInputs(q, k, v, pos_offset)


def seeded_pattern(n_layers: int, n_full: int, seed: int) -> str:
    """A layer pattern with exactly n_full 'F' characters: layer 0 plus
    n_full - 1 layers drawn from a seeded permutation of layers 1..n_layers-1."""
    if not 1 <= n_full <= n_layers:
        raise ValueError("n_full out of range")
    rng = np.random.default_rng(seed)
    rest = rng.permutation(np.arange(1, n_layers))[: n_full - 1]
    chars = ["S"] * n_layers
    chars[0] = "F"
    for l in rest:
        chars[int(l)] = "F"
    return "".join(chars)


@dataclass
class PagedLayout:
    """A paged, ragged decode cache layout. seq_lens: int32 [B] (may hold values
    outside [0, max_seq_len] to exercise clamping); block_table: int32
    [B, max_pages], request b's pages in order, entries it does not use = -1."""
    seq_lens: torch.Tensor
    block_table: torch.Tensor
    page_size: int
    num_pages: int
    max_seq_len: int

    def to(self, device) -> "PagedLayout":
        return PagedLayout(self.seq_lens.to(device), self.block_table.to(device), self.page_size,
                           self.num_pages, self.max_seq_len)


def make_paged_layout(seq_lens, page_size: int, max_seq_len: int, *, seed: int,
                      spare_pages: int = 3) -> PagedLayout:
    """Request b gets ceil(min(max(seq_lens[b], 0), max_seq_len) / page_size)
    pages; all pages of the pool (plus spare_pages nobody uses) are handed out in
    the order of a seeded permutation, so neighbouring tokens of a request sit
    in unrelated pages."""
    lens = [int(x) for x in seq_lens]
    max_pages = -(-max_seq_len // page_size)
    need = [-(-min(max(n, 0), max_seq_len) // page_size) for n in lens]
    num_pages = sum(need) + spare_pages
    perm = np.random.default_rng(seed).permutation(num_pages)
    bt = np.full((len(lens), max_pages), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[at:at + n]
        at += n
    return PagedLayout(torch.tensor(lens, dtype=torch.int32), torch.from_numpy(bt), page_size, num_pages,
                       max_seq_len)


def scatter_to_pages(flat: torch.Tensor, layout: PagedLayout, junk: torch.Tensor) -> torch.Tensor:
    """Page pool [num_pages, page_size, ...] holding flat[b, s] ([B, max_seq_len,
    ...]) at request b's token s for every s below its clamped length; every
    other slot keeps the value of junk (same shape as the pool)."""
    pool = junk.clone()
    bt = layout.block_table.cpu()
    for b in range(flat.shape[0]):
        n = min(max(int(layout.seq_lens[b]), 0), layout.max_seq_len)
        for s in range(0, n, layout.page_size):
            m = min(layout.page_size, n - s)
            pool[int(bt[b, s // layout.page_size]), :m] = flat[b, s:s + m].to(pool.device)
    return pool


def make_correlated_topk(n_layers: int, rows: int, k: int, n_k: int, *, swap: float, seed: int,
                         reset_every: int = 0, short_rows: int = 0) -> np.ndarray:
    """Synthetic per-layer top-k index rows [n_layers, rows, k] int32 whose
    layers overlap like a random walk: layer 0's row is a random k-subset of
    [0, n_k), and layer l's row is layer l-1's with round(swap * k) entries
    replaced by fresh random tokens (a fresh subset every reset_every layers,
    if > 0). The first short_rows rows hold only their row number + 1 <= k
    valid entries (a causal prefix), padded with -1. Rows list their tokens in
    random order."""
    rng = np.random.default_rng(seed)
    out = np.full((n_layers, rows, k), -1, dtype=np.int32)
    m = int(round(swap * k))
    for r in range(rows):
        cnt = min(k, r + 1) if r < short_rows else k
        pool = min(n_k, r + 1) if r < short_rows else n_k
        cur = None
        for l in range(n_layers):
            if cur is None or (reset_every and l % reset_every == 0):
                cur = rng.choice(pool, cnt, replace=False)
            elif m and cnt < pool:
                cur = cur.copy()
                drop = rng.choice(cnt, min(m, cnt), replace=False)
                fresh = np.setdiff1d(rng.choice(pool, min(pool, cnt + 2 * m), replace=False), cur)
                take = min(len(drop), len(fresh))
                cur[drop[:take]] = fresh[:take]
            out[l, r, :cnt] = rng.permutation(cur)
    return out


def host_bits(t: Optional[torch.Tensor]):
    """Raw bits of a tensor as a numpy array on the host: bf16 -> uint16,
    float8_e4m3fn -> uint8, fp32 -> float32, int32 -> int32."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype in (torch.float32, torch.int32, torch.int64, torch.float64):
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")
