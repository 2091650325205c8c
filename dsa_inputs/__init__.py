"""Seeded synthetic inputs for the DSA indexer / top-k / sparse-attention path.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It only *draws* inputs (random numbers, dtype casts of those draws,
seeded layer patterns, paged cache layouts); it contains none of the method's
arithmetic, so the two sides that are compared never share a computation.

Seed rule: seed = 1_000_000 * config + 1000 * layer + tensor_id, with the
tensor ids below. Every tensor is drawn from its own generator, so a layer or
tensor can be regenerated alone.
"""
from .gen import (  # noqa: F401
    TENSOR_IDS,
    seed_for,
    randn,
    IndexerInputs,
    AttnInputs,
    make_indexer_inputs,
    make_attn_inputs,
    make_int_indexer_inputs,
    seeded_pattern,
    PagedLayout,
    make_paged_layout,
    scatter_to_pages,
    make_correlated_topk,
    to_e4m3_clipped,
    host_bits,
)
