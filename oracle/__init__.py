"""CPU oracle for the DSA lightning indexer, per-query top-k, sparse attention
and the IndexCache F/S layer stack.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does, and this
package imports nothing from the product path. Everything here is plain NumPy
in float64 (and pure Python for the brute-force references), reading the exact
bits of the device inputs.

Sources. The method comes from "IndexCache: Accelerating Sparse Attention via
Cross-Layer Index Reuse" (arXiv 2603.12201): the abstract (indexer -> top-k ->
sparse core attention; Full and Shared layers), the paper's Figure 2 caption
(the single cached index tensor overwritten at each F layer) and the IndexCache
repository README ("Option A - Uniform interleaving", "Option B - Custom
pattern", "Default behavior"). The pages name the lightning indexer but do not
print its formula; the oracle uses the standard DSA indexer score
I[t,s] = sum_j w[t,j] * ReLU(q[t,j,:] . k[s,:]) over causal s <= pos(t).

Pinning status (what each function is checked against, besides itself):
  formats.bf16_to_f64        torch's bfloat16 -> float64 conversion (library)
  formats.e4m3fn_table       torch's float8_e4m3fn conversion (library) + format
                             extremes (448, 2**-9)
  indexer.indexer_scores     pure-Python brute force; exact-integer inputs; closed
                             forms (positive inputs -> plain GEMM); fp8 scale
                             homogeneity; hand-worked golden example
  indexer.topk_from_scores   brute-force full sort; hand-worked golden example;
                             short-row and all-ties invariants
  attention.sparse_attention textbook dense causal attention via torch's
                             scaled_dot_product_attention (k >= L); mean-of-V
                             (q = 0); single selected row; hand-worked example
  pattern.resolve_pattern    README examples (freq 2, freq 4, GLM-5 string, default)
  stack.run_stack            cached-index invariants (S == preceding F, all-F ==
                             per layer, freq 1 == default)
  quant.e4m3fn_encode        torch's float32 -> float8_e4m3fn cast (library) on
                             grids with every midpoint; extremes
  quant.quantize_rows_fp8    the row maximum maps to +-448; dequantisation error
                             within half a step; zero rows
  paged.*                    the flat functions per request on pools built by
                             scattering flat rows; junk outside the context;
                             page renaming; length clamping; append
No function is "parity unpinned".
"""
from .formats import bf16_to_f64, e4m3fn_table, e4m3fn_to_f64  # noqa: F401
from .indexer import (  # noqa: F401
    indexer_scores,
    indexer_scores_rows,
    topk_from_scores,
    indexer_topk,
    score_order_key,
)
from .attention import sparse_attention, sparse_attention_rows  # noqa: F401
from .pattern import resolve_pattern, PatternError  # noqa: F401
from .stack import run_stack  # noqa: F401
from .quant import e4m3fn_encode, quantize_rows_fp8  # noqa: F401
from . import paged  # noqa: F401
