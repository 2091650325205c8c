/*
 * dsa.h - C ABI of libdsa: the DeepSeek-Sparse-Attention hot path on AMD
 * Instinct MI355X (gfx950): the lightning indexer fused with per-query top-k
 * selection, sparse attention over the selected tokens, and the IndexCache
 * layer stack in which Full (F) layers compute the indices and Shared (S)
 * layers reuse them.
 *
 * Sources.
 *  - "IndexCache: Accelerating Sparse Attention via Cross-Layer Index Reuse"
 *    (arXiv 2603.12201), Abstract: a lightweight lightning indexer picks the
 *    top-k tokens for each query and core attention runs over those tokens
 *    only (O(L*k) instead of O(L^2)); the indexer itself stays O(L^2) and runs
 *    at every layer; IndexCache lets Shared layers reuse the indices of a Full
 *    layer.
 *  - Same paper, Figure 2 caption: one conditional branch in the layer loop;
 *    the cached index tensor is a temporary buffer holding only the current
 *    indices, overwritten at each F layer, needing no memory beyond plain DSA.
 *  - IndexCache repository README, "Step 3: Launch with IndexCache": the two
 *    configuration keys index_topk_freq (Option A, uniform interleaving) and
 *    index_topk_pattern (Option B, one 'F'/'S' character per DSA layer), and
 *    "Default behavior" (neither key: every layer runs its indexer).
 * The pages name the indexer but do not print its formula; this library
 * computes the standard DSA indexer score
 *      I[t,s] = sum_j w[t,j] * ReLU( q[t,j,:] . k[s,:] ),  0 <= s <= pos(t),
 * where pos(t) = q_pos_offset + t. For fp8 inputs the dequantised operands are
 * e4m3(q)*q_scale[t] and e4m3(k)*k_scale[s].
 *
 * Conventions (every function):
 *  - Ownership: the caller owns every device buffer and the stream. The
 *    library allocates no device memory and keeps no device state; scratch
 *    space is the caller's workspace, sized by the *_workspace_size calls.
 *  - Layouts: every tensor is dense row-major with the last dimension
 *    contiguous, exactly in the shapes documented below (no strides).
 *  - Pointers are device pointers unless stated; they must be aligned to
 *    16 bytes (workspace: 256 bytes).
 *  - Execution: asynchronous on `stream` (a hipStream_t passed as void*,
 *    NULL = the null stream); nothing synchronises inside the library.
 *  - Validation happens on the host before the first HIP call: on any error
 *    the call returns a status, sets dsa_last_error() (thread-local text) and
 *    touches no output.
 *  - Index outputs are int32, in rank order (higher score first, equal
 *    scores by lower index first; -0.0 equals +0.0), padded with -1 when a
 *    query has fewer than topk causal keys.
 *  - Sizes are validated in 64-bit arithmetic; every element count must fit
 *    in int64 and every per-dimension size in int32.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, bad size, misaligned pointer */
  DSA_ERR_UNSUPPORTED = 2,      /* shape or dtype outside the supported set   */
  DSA_ERR_BAD_PATTERN = 3,      /* index_topk_pattern string rejected         */
  DSA_ERR_WORKSPACE = 4,        /* workspace missing or too small             */
  DSA_ERR_HIP = 5               /* a HIP runtime call or launch failed        */
} dsa_status;

typedef enum {
  DSA_BF16 = 0,        /* bfloat16 q_idx / k_idx                               */
  DSA_FP8_E4M3FN = 1   /* OCP fp8 e4m3fn q_idx / k_idx + fp32 per-token scales */
} dsa_dtype;

/* Indexer + top-k for B independent sequences (prefill) or requests (decode).
 *
 *   q        [B, n_q, n_heads, head_dim]  bf16 or e4m3fn (query-side indexer
 *                                          vectors, one per indexer head)
 *   k        [B, n_k, head_dim]           same dtype (indexer keys)
 *   w        [B, n_q, n_heads]            fp32 per-query head weights
 *   q_scale  [B, n_q] fp32, k_scale [B, n_k] fp32: fp8 only (> 0), NULL for bf16
 *   out_idx  [B, n_q, topk] int32          selected key indices, rank order
 *   out_scores [B, n_q, topk] fp32         optional (NULL): score of each
 *                                          selected key (-inf where idx = -1)
 *   debug_full_scores [B, n_q, n_k] fp32   optional (NULL), test mode: the
 *                                          same kernel also stores every causal
 *                                          score it computes (non-causal
 *                                          entries are left untouched)
 * Query t of a sequence sits at position q_pos_offset + t and sees keys
 * 0..min(q_pos_offset + t, n_k - 1). Requires 0 <= q_pos_offset and
 * q_pos_offset + n_q <= n_k. n_q == 1 selects the decode path (the one query's
 * keys are spread over the whole GPU); n_q > 1 the prefill path.
 * Supported: n_heads in 1..64, head_dim in {32, 64, 128} (fp8: {64, 128}),
 * topk in 1..2048. */
typedef struct {
  uint32_t struct_size;         /* = sizeof(dsa_indexer_args) */
  int32_t B, n_q, n_k, q_pos_offset;
  int32_t n_heads, head_dim, topk;
  int32_t dtype;                /* dsa_dtype */
  const void *q;
  const void *k;
  const float *w;
  const float *q_scale;
  const float *k_scale;
  int32_t *out_idx;
  float *out_scores;
  float *debug_full_scores;
  void *workspace;
  size_t workspace_bytes;
  /* Optional (NULL): HOST array of 3 hipEvent_t (as void*) recorded on the
   * stream before the score kernel, between the score kernel and the
   * selection kernels, and after the last kernel, so that a caller can time
   * the phases without a profiler. */
  void *const *phase_events;
} dsa_indexer_args;

/* Sparse attention over given indices, one KV head shared by n_heads query
 * heads (bf16 in, fp32 softmax, bf16 out).
 *
 *   q    [B, n_q, n_heads, head_dim] bf16;  k, v [B, n_k, head_dim] bf16
 *   idx  [B, n_q, topk] int32: entries < 0, > q_pos_offset + t or >= n_k are
 *        skipped (so -1 padding is ignored); duplicates count once each
 *   out  [B, n_q, n_heads, head_dim] bf16 (softmax-normalised)
 *   lse  [B, n_q, n_heads] fp32, optional (NULL): natural-log sum-exp of the
 *        scaled scores (-inf and out = 0 for a query with no valid entry)
 * scale = 0 means 1/sqrt(head_dim). Supported: n_heads in 1..16, head_dim in
 * {64, 128}, topk in 1..4096. */
typedef struct {
  uint32_t struct_size;         /* = sizeof(dsa_attn_args) */
  int32_t B, n_q, n_k, q_pos_offset;
  int32_t n_heads, head_dim, topk;
  float scale;
  const void *q;
  const void *k;
  const void *v;
  const int32_t *idx;
  void *out;
  float *lse;
  void *workspace;
  size_t workspace_bytes;
  /* Optional (NULL): HOST array of 2 hipEvent_t recorded before the first and
   * after the last attention kernel. */
  void *const *phase_events;
} dsa_attn_args;

/* A stack of n_layers DSA layers, each = (indexer + top-k if F) + sparse
 * attention, with one shared index buffer (the IndexCache cache).
 *
 * `indexer` and `attn` give the shapes and dtype shared by all layers; their
 * pointer, workspace and phase_events fields are ignored. The per-layer pointers
 * are HOST arrays of n_layers DEVICE pointers. q_scale / k_scale arrays are
 * required for fp8 and must be NULL for bf16. lse may be NULL (no lse) or an
 * array whose entries may be NULL. out entries may alias each other.
 * idx_buf [B, n_q, topk] int32 is the single cached index tensor: every F
 * layer overwrites it, every S layer reads it; after the call it holds the
 * indices of the last F layer. layer_events, if not NULL, is a host array of
 * n_layers + 1 hipEvent_t (as void*): event l is recorded before layer l and
 * event n_layers after the last layer. The workspace size does not depend on
 * the pattern. */
typedef struct {
  uint32_t struct_size;         /* = sizeof(dsa_stack_args) */
  int32_t n_layers;
  dsa_indexer_args indexer;
  dsa_attn_args attn;
  const void *const *q_idx;
  const void *const *k_idx;
  const float *const *w;
  const float *const *q_scale;
  const float *const *k_scale;
  const void *const *q;
  const void *const *k;
  const void *const *v;
  void *const *out;
  float *const *lse;
  int32_t *idx_buf;
  void *const *layer_events;
  void *workspace;
  size_t workspace_bytes;
} dsa_stack_args;

/* Paged, ragged decode: the KV layout a serving engine keeps. One query token
 * per request; request b's context holds seq_lens[b] tokens, the new token
 * being the last (position seq_lens[b] - 1), and token s of request b lives
 * in page block_table[b * max_pages + s / page_size], slot s % page_size, of a
 * page pool. Pools: indexer keys [num_pages, page_size, head_dim] (indexer
 * dtype), their fp8 scales [num_pages, page_size] fp32, attention K and V
 * [num_pages, page_size, head_dim] bf16.
 *   seq_lens    device int32 [B]; values are clamped to [0, max_seq_len]. A
 *               request with no tokens gets all -1 indices (attention: out 0,
 *               lse -inf).
 *   block_table device int32 [B, max_pages]; the entries of the pages a request
 *               uses must lie in [0, num_pages). Other entries are not read.
 *               An out-of-range entry is clamped into the pool: that request's
 *               results are then unspecified, but no access leaves the pool.
 *   page_size   a multiple of 32; max_pages * page_size >= max_seq_len.
 * Indices are logical token positions, so the IndexCache buffer (one index
 * tensor reused by the S layers, paper listing page, Figure 2 caption) needs
 * no change under paging. */
typedef struct {
  uint32_t struct_size;         /* = sizeof(dsa_paged_kv) */
  int32_t max_seq_len;          /* host upper bound of seq_lens: sizes grids and workspaces */
  int32_t page_size, max_pages, num_pages;
  const int32_t *seq_lens;
  const int32_t *block_table;
} dsa_paged_kv;

/* DSA_ABI_VERSION of the built library. */
int32_t dsa_abi_version(void);

/* Bytes of workspace the matching call needs (0 is possible). Validates the
 * shape fields only; pointers may be NULL. */
dsa_status dsa_indexer_workspace_size(const dsa_indexer_args *args, size_t *bytes);
dsa_status dsa_attn_workspace_size(const dsa_attn_args *args, size_t *bytes);
dsa_status dsa_stack_workspace_size(const dsa_stack_args *args, size_t *bytes);

/* Resolves the IndexCache layer pattern (README, Options A and B and Default
 * behavior) into out[0..n_layers) of 'F'/'S' plus a terminating NUL (out is a
 * HOST buffer of n_layers + 1 bytes). Rules:
 *   pattern != NULL: length n_layers, characters 'F'/'S' only (case
 *                    sensitive), first character 'F'   -> else BAD_PATTERN
 *   index_topk_freq > 0: layer l is F iff l % freq == 0 (layer 0 is F)
 *   neither set: every layer is F
 *   both set, freq < 0 or n_layers < 1: INVALID_ARGUMENT.
 * Pure host code; needs no GPU. */
dsa_status dsa_resolve_pattern(int32_t n_layers, const char *pattern, int32_t index_topk_freq,
                               char *out);

/* The indexer scores of every causal (query, key) pair followed by the exact
 * per-query top-k of those scores (rank order, -1 padded). The L x L score
 * matrix is never stored (except in debug_full_scores test mode). */
dsa_status dsa_indexer_scores_topk(const dsa_indexer_args *args, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as dsa_indexer_scores_topk, with the library's own scratch in
 * place of a workspace. args->workspace must be NULL and workspace_bytes 0.
 * The scratch is a static device array of DSA_STATIC_SCRATCH_BYTES (64 MiB)
 * that each GPU holds from the first call on it until the process ends; a
 * shape whose dsa_indexer_workspace_size exceeds it returns DSA_ERR_WORKSPACE
 * before anything is enqueued (e.g. decode of B = 32 requests over 200K-token
 * contexts at topk = 2048 needs about 32 MB; prefill needs about 64 KB per
 * query row at topk = 2048). The call allocates nothing, on the device or
 * through any library. Every call on one GPU shares that GPU's scratch and
 * the scratch keeps the last call's contents (the kernels initialise what
 * they read): calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller. The first call on a
 * device looks up the array's device address (hipGetSymbolAddress); a
 * failure there is DSA_ERR_HIP. */
#define DSA_STATIC_SCRATCH_BYTES (64u << 20)
dsa_status dsa_indexer_scores_topk_static(const dsa_indexer_args *args, void *stream);

/* Softmax attention of every query head over the key/value rows listed in idx. */
dsa_status dsa_sparse_attn(const dsa_attn_args *args, void *stream);

/* Runs the layer stack: layer l runs the indexer into idx_buf iff the resolved
 * pattern (pattern string, or index_topk_freq, or neither = all F) has 'F' at
 * l, then sparse attention of layer l over idx_buf. Arguments are validated
 * for every layer before anything is enqueued. */
dsa_status dsa_layer_stack_run(const dsa_stack_args *args, const char *pattern,
                               int32_t index_topk_freq, void *stream);

/* Chunked prefill of one sequence through the layer stack: a long prompt is
 * prefilled in chunks of query rows over the keys cached so far (the prefill
 * columns of the paper's Table 1 reach 200K tokens; a serving engine splits
 * such prompts). args describe the whole prefill of one sequence (B = 1):
 * n_q query rows at positions q_pos_offset .. q_pos_offset + n_q - 1 over n_k
 * keys. Chunk c covers rows [c * chunk_rows, min((c + 1) * chunk_rows, n_q))
 * and runs the whole stack exactly as dsa_layer_stack_run would with those
 * rows as its queries and the keys up to the chunk's last position (the
 * cached prefix plus the chunk) as n_k. Each chunk writes its own rows of
 * out[l] (and lse[l]); the per-layer query inputs (q_idx, w, q_scale, q) are
 * read at the chunk's rows; k_idx, k_scale, k and v are read as given.
 * idx_buf is the per-chunk index cache, [chunk_rows, topk] int32: each F
 * layer of a chunk overwrites its first rows, each S layer reuses them, and
 * after the call it holds the last chunk's last F layer's indices. The
 * results equal one dsa_layer_stack_run over all rows: the indices of every
 * row bit for bit, and the attention outputs bit for bit when every chunk,
 * like the whole run, has more than 1024 rows (each row is then handled by
 * one wave in both runs), within rounding otherwise. The workspace
 * (dsa_chunked_stack_workspace_size) is sized for one chunk, not the whole
 * prompt. layer_events must be NULL. B != 1, chunk_rows < 1 or
 * layer_events set: UNSUPPORTED / INVALID_ARGUMENT, before
 * anything is enqueued; any other error is reported before the first chunk
 * is enqueued. */
dsa_status dsa_chunked_stack_workspace_size(const dsa_stack_args *args, int32_t chunk_rows, size_t *bytes);
dsa_status dsa_layer_stack_run_chunked(const dsa_stack_args *args, int32_t chunk_rows, const char *pattern,
                                       int32_t index_topk_freq, void *stream);

/* Decode indexer + top-k over a paged, ragged cache. args as for
 * dsa_indexer_scores_topk with n_q = 1 and n_k = kv->max_seq_len (q_pos_offset
 * is ignored: request b's query sits at seq_lens[b] - 1); k and k_scale point
 * at the page pools; debug_full_scores, if given, is [B, max_seq_len] (entries
 * at or past a request's length are left untouched). out_idx holds logical
 * token positions. The workspace is dsa_indexer_workspace_size of args. */
dsa_status dsa_paged_indexer_topk(const dsa_indexer_args *args, const dsa_paged_kv *kv, void *stream);

/* Decode sparse attention over a paged cache. args as for dsa_sparse_attn with
 * n_q = 1 and n_k = kv->max_seq_len; k and v point at the page pools; idx holds
 * logical positions (entries < 0 or >= seq_lens[b] are skipped). The workspace
 * is dsa_attn_workspace_size of args. */
dsa_status dsa_paged_sparse_attn(const dsa_attn_args *args, const dsa_paged_kv *kv, void *stream);

/* The layer stack of one decode step over paged caches: as
 * dsa_layer_stack_run with n_q = 1, n_k = kv->max_seq_len, every per-layer
 * k_idx, k_scale, k and v pointer a page pool (all layers share kv), and
 * idx_buf [B, topk] holding logical positions. */
dsa_status dsa_paged_layer_stack_run(const dsa_stack_args *args, const dsa_paged_kv *kv, const char *pattern,
                                     int32_t index_topk_freq, void *stream);

/* Writes src[b] (row_bytes bytes) to its request's last position
 * seq_lens[b] - 1 in a page pool [num_pages, page_size, row_bytes]: the step
 * before the path, run for the new token's indexer key (and fp8 scale), K and
 * V. Requests with seq_lens[b] < 1 are skipped. row_bytes is a positive
 * multiple of 4; src and pool are 4-byte aligned device pointers. */
dsa_status dsa_paged_append_rows(const void *src, int32_t B, int32_t row_bytes, void *pool,
                                 const dsa_paged_kv *kv, void *stream);

/* Per-token fp8 quantisation of indexer inputs: the step that produces the
 * fp8 e4m3 q_idx / k_idx with per-token fp32 scales that the long-context
 * configuration feeds dsa_indexer_scores_topk (IndexCache paper page,
 * configuration of the 200K fp8 runs; the pages do not give the quantiser).
 * For each row r of x (bf16, [rows, cols] row-major; a token's values: for
 * q_idx [B, n_q, H, D] one row is one query token, cols = H * D, for k_idx one
 * key token, cols = D):
 *   amax = max_c |x[r,c]|, scale[r] = fl32(amax / 448) (1 if amax == 0),
 *   out[r,c] = e4m3fn(fl32(x[r,c] / scale[r])), round to nearest, ties to the
 *              even mantissa, magnitudes above 448 clamped to 448 (never NaN),
 * fl32 = IEEE binary32 rounding. Dequantisation is e4m3fn(out) * scale.
 * x: device, 16-byte aligned; out: device [rows, cols] bytes (OCP e4m3fn codes),
 * 8-byte aligned; scale: device [rows] fp32. rows >= 0 (0 = nothing to do);
 * cols a positive multiple of 8, at most 1 << 24. Inputs must be finite.
 * Asynchronous on stream; on a validation error nothing is written. */
dsa_status dsa_quantize_fp8_rows(const void *x, int64_t rows, int32_t cols, void *out, float *scale,
                                 void *stream);

/* Cross-layer top-k overlap, the measurement behind IndexCache (paper
 * appendix, Figure 4: pairwise overlap of the layers' top-k index sets; the
 * repository page's "Key Insight": adjacent layers share most of theirs).
 *   idx    device int32 [n_layers, rows, topk]: row r of layer l lists the
 *          selected tokens of the same query r in every layer (e.g. the
 *          indexer's out_idx per layer). Entries < 0 or >= n_k are ignored;
 *          the valid entries of a row must be distinct (as the indexer's are).
 *   inter  device int64 [n_layers, n_layers], overwritten:
 *          inter[a][b] = sum_r |S_a(r) & S_b(r)|, S_l(r) the valid entries of
 *          row r of layer l; inter[a][a] = sum_r |S_a(r)|. The overlap ratio
 *          of a and b is inter[a][b] / inter[a][a].
 * 1 <= n_layers <= 1024, rows >= 1, topk >= 1, 1 <= n_k <= 2^19 (one bit per
 * token in LDS), else INVALID_ARGUMENT / UNSUPPORTED. Asynchronous on stream. */
dsa_status dsa_topk_overlap(const int32_t *idx, int32_t n_layers, int32_t rows, int32_t topk, int32_t n_k,
                            int64_t *inter, void *stream);

/* Similarity-based layer pattern from an overlap matrix (the training-free
 * "similarity-based searched pattern" of the paper's Table 5; the pages do
 * not give the search, the plain reading is taken): among the patterns with
 * n_full F layers, layer 0 always F, the one that maximises
 *   sum over S layers l of inter[f(l)][l],  f(l) = the last F layer before l
 * (the layer whose cached indices l reuses, paper Figure 2 caption), i.e. the
 * number of selections each S layer shares with its source. The optimum is
 * exact (a segment recursion, O(n_full * n_layers^2)); among equal totals the
 * lexicographically smallest list of F layers wins. inter: HOST int64
 * [n_layers, n_layers] with entries in 0..2^52 (dsa_topk_overlap's output);
 * out: HOST buffer of n_layers + 1 bytes ('F'/'S' string, NUL-terminated),
 * usable as dsa_layer_stack_run's pattern. Pure host code; needs no GPU. */
dsa_status dsa_similarity_pattern(int32_t n_layers, const int64_t *inter, int32_t n_full, char *out);

/* Static text of a status code. */
const char *dsa_status_string(dsa_status status);

/* Thread-local detail of the last failed call on this thread ("" if none). */
const char *dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
