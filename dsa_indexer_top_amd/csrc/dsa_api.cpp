// Host side of libdsa: argument validation, IndexCache pattern resolution,
// workspace sizing and kernel dispatch. Every check runs before the first HIP
// call, so an invalid call touches no output and needs no GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>
#include <string>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status ok() {
  g_last_error.clear();
  return DSA_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool count4(int64_t a, int64_t b, int64_t c, int64_t d, int64_t* out) {
  int64_t x, y;
  return mul_ok(a, b, &x) && mul_ok(x, c, &y) && mul_ok(y, d, out);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxTopk = 2048;
constexpr int kMaxAttnTopk = 4096;
constexpr int kMaxB = 65535;
constexpr int kMaxOverlapLayers = 1024;
constexpr int kMaxOverlapKeys = 1 << 19;  // 64 KB of LDS bitmap

dsa_status check_indexer_shape(const dsa_indexer_args* a, const char* what) {
  if (!a) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: args is NULL", what);
  if (a->struct_size != sizeof(dsa_indexer_args))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu", what, a->struct_size,
                sizeof(dsa_indexer_args));
  if (a->B < 1 || a->B > kMaxB) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: B=%d out of 1..%d", what, a->B, kMaxB);
  if (a->n_q < 1 || a->n_k < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: n_q=%d n_k=%d must be >= 1", what, a->n_q, a->n_k);
  if (a->q_pos_offset < 0 || (int64_t)a->q_pos_offset + a->n_q > a->n_k)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: need 0 <= q_pos_offset and q_pos_offset + n_q <= n_k (%d + %d vs %d)",
                what, a->q_pos_offset, a->n_q, a->n_k);
  if (a->dtype != DSA_BF16 && a->dtype != DSA_FP8_E4M3FN)
    return fail(DSA_ERR_UNSUPPORTED, "%s: dtype %d unsupported", what, a->dtype);
  if (a->n_heads < 1 || a->n_heads > 64)
    return fail(DSA_ERR_UNSUPPORTED, "%s: n_heads=%d outside 1..64", what, a->n_heads);
  const int d = a->head_dim;
  const bool d_ok = a->dtype == DSA_BF16 ? (d == 32 || d == 64 || d == 128) : (d == 64 || d == 128);
  if (!d_ok) return fail(DSA_ERR_UNSUPPORTED, "%s: head_dim=%d unsupported for this dtype", what, d);
  if (a->topk < 1 || a->topk > kMaxTopk)
    return fail(DSA_ERR_UNSUPPORTED, "%s: topk=%d outside 1..%d", what, a->topk, kMaxTopk);
  int64_t n;
  if (!count4(a->B, a->n_q, a->n_heads, a->head_dim, &n) || !count4(a->B, a->n_q, a->n_k, 1, &n) ||
      !count4(a->B, a->n_q, dsa::cand_capacity(a->topk, a->n_q == 1), 8, &n))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: sizes overflow int64", what);
  return DSA_OK;
}

dsa_status check_attn_shape(const dsa_attn_args* a, const char* what) {
  if (!a) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: args is NULL", what);
  if (a->struct_size != sizeof(dsa_attn_args))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu", what, a->struct_size,
                sizeof(dsa_attn_args));
  if (a->B < 1 || a->B > kMaxB) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: B=%d out of 1..%d", what, a->B, kMaxB);
  if (a->n_q < 1 || a->n_k < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: n_q=%d n_k=%d must be >= 1", what, a->n_q, a->n_k);
  if (a->q_pos_offset < 0 || (int64_t)a->q_pos_offset + a->n_q > a->n_k)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: need 0 <= q_pos_offset and q_pos_offset + n_q <= n_k", what);
  if (a->n_heads < 1 || a->n_heads > 16)
    return fail(DSA_ERR_UNSUPPORTED, "%s: n_heads=%d outside 1..16", what, a->n_heads);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "%s: head_dim=%d unsupported (64, 128)", what, a->head_dim);
  if (a->topk < 1 || a->topk > kMaxAttnTopk)
    return fail(DSA_ERR_UNSUPPORTED, "%s: topk=%d outside 1..%d", what, a->topk, kMaxAttnTopk);
  if (!(a->scale >= 0.0f) || a->scale > 3.0e38f)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: scale must be finite and >= 0", what);
  int64_t n;
  if (!count4(a->B, a->n_q, a->n_heads, a->head_dim, &n) || !count4(a->B, a->n_q, a->topk, 1, &n) ||
      !count4(a->B, a->n_k, a->head_dim, 1, &n))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: sizes overflow int64", what);
  return DSA_OK;
}

dsa_status check_indexer_ptrs(const dsa_indexer_args* a, const void* q, const void* k, const float* w,
                              const float* qs, const float* ks, const int32_t* out_idx, const char* what) {
  if (!q || !k || !w || !out_idx) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: q, k, w and out_idx are required", what);
  if (a->dtype == DSA_FP8_E4M3FN && (!qs || !ks))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: fp8 needs q_scale and k_scale", what);
  if (a->dtype == DSA_BF16 && (qs || ks))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: q_scale/k_scale must be NULL for bf16", what);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(out_idx, 4) ||
      (qs && !aligned(qs, 4)) || (ks && !aligned(ks, 4)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: misaligned pointer (q, k: 16 bytes; others: 4)", what);
  return DSA_OK;
}

dsa_status check_attn_ptrs(const void* q, const void* k, const void* v, const int32_t* idx, const void* out,
                           const float* lse, const char* what) {
  if (!q || !k || !v || !idx || !out) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: q, k, v, idx and out are required", what);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(idx, 4) || !aligned(out, 4) ||
      (lse && !aligned(lse, 4)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: misaligned pointer (q, k, v: 16 bytes; others: 4)", what);
  return DSA_OK;
}

dsa_status check_workspace(void* ws, size_t have, size_t need, const char* what) {
  if (need == 0) return DSA_OK;
  if (!ws) return fail(DSA_ERR_WORKSPACE, "%s: workspace is NULL but %zu bytes are needed", what, need);
  if (have < need) return fail(DSA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", what, have, need);
  if (!aligned(ws, 256)) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", what);
  return DSA_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

dsa::IndexerParams make_indexer_params(const dsa_indexer_args* a, const void* q, const void* k, const float* w,
                                       const float* qs, const float* ks, int32_t* out_idx, float* out_scores,
                                       float* dump, void* ws) {
  dsa::IndexerParams p;
  memset(&p, 0, sizeof(p));
  p.B = a->B;
  p.n_q = a->n_q;
  p.n_k = a->n_k;
  p.pos_offset = a->q_pos_offset;
  p.H = a->n_heads;
  p.D = a->head_dim;
  p.topk = a->topk;
  p.fp8 = a->dtype == DSA_FP8_E4M3FN;
  p.q = q;
  p.k = k;
  p.w = w;
  p.q_scale = qs;
  p.k_scale = ks;
  p.out_idx = out_idx;
  p.out_scores = out_scores;
  p.dump = dump;
  p.ev = nullptr;
  dsa::indexer_bind_workspace(p, ws);
  return p;
}

dsa::AttnParams make_attn_params(const dsa_attn_args* a, const void* q, const void* k, const void* v,
                                 const int32_t* idx, void* out, float* lse, void* ws) {
  dsa::AttnParams p;
  memset(&p, 0, sizeof(p));
  p.B = a->B;
  p.n_q = a->n_q;
  p.n_k = a->n_k;
  p.pos_offset = a->q_pos_offset;
  p.H = a->n_heads;
  p.D = a->head_dim;
  p.topk = a->topk;
  p.scale = a->scale > 0.0f ? a->scale : 1.0f / sqrtf((float)a->head_dim);
  p.q = q;
  p.k = k;
  p.v = v;
  p.idx = idx;
  p.out = out;
  p.lse = lse;
  p.nsplit = dsa::attn_nsplit(a->B, a->n_q, a->topk);
  p.part = (float*)ws;
  p.ev = nullptr;
  return p;
}

dsa_status run_indexer(const dsa::IndexerParams& p, hipStream_t s) {
  const hipError_t e = p.n_q == 1 ? dsa::launch_indexer_decode(p, s) : dsa::launch_indexer_prefill(p, s);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "indexer launch failed: %s", hipGetErrorString(e));
  return DSA_OK;
}

dsa_status run_attn(const dsa::AttnParams& p, hipStream_t s) {
  const hipError_t e = dsa::launch_sparse_attn(p, s);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "sparse attention launch failed: %s", hipGetErrorString(e));
  return DSA_OK;
}

}  // namespace

namespace dsa {

// Byte offset of the decode plan (followed by the histograms) in the indexer
// workspace of a decode call (n_q == 1): after the candidate lists and keys.
size_t indexer_decode_plan_offset(int B, int n_k, int topk) {
  const size_t C = (size_t)cand_capacity(topk, true);
  return 2 * round_up((size_t)B * C * 4, 256) + (size_t)B * decode_key_stride(n_k) * 4;
}

size_t indexer_workspace_bytes(int B, int n_q, int n_k, int topk) {
  const size_t rows = (size_t)B * n_q;
  const size_t C = (size_t)cand_capacity(topk, n_q == 1);
  size_t sz = 0;
  sz += round_up(rows * C * 4, 256);  // cand_key
  sz += round_up(rows * C * 4, 256);  // cand_idx
  if (n_q == 1) {
    sz += (size_t)B * decode_key_stride(n_k) * 4;                    // decode keys
    sz += round_up(((size_t)B + kDecodeTargetBlocks) * 3 * 4, 256);  // ragged-decode block plan
    sz += (size_t)B * kDecodeHistRow * 4;  // decode histograms and counters
  } else {
    sz += round_up(rows * 4, 256);  // cand_cnt
  }
  return sz;
}

void indexer_bind_workspace(IndexerParams& p, void* ws) {
  const size_t rows = (size_t)p.B * p.n_q;
  p.C = cand_capacity(p.topk, p.n_q == 1);
  char* c = (char*)ws;
  p.cand_key = (uint32_t*)c;
  c += round_up(rows * p.C * 4, 256);
  p.cand_idx = (int32_t*)c;
  c += round_up(rows * p.C * 4, 256);
  if (p.n_q == 1) {
    p.dec_keys = (uint32_t*)c;
    c += (size_t)p.B * decode_key_stride(p.n_k) * 4;
    p.dec_work = (int32_t*)c;
    c += round_up(((size_t)p.B + kDecodeTargetBlocks) * 3 * 4, 256);
    p.dec_hist = (uint32_t*)c;
    p.cand_cnt = (int32_t*)(p.dec_hist + kDecodeCntOffset);
    p.cnt_stride = kDecodeHistRow;
  } else {
    p.cand_cnt = (int32_t*)c;
    p.cnt_stride = 1;
  }
}

int attn_nsplit(int B, int n_q, int topk) {
  // about 2048 waves over the whole call (the best measured from one decode
  // request to 16K prefill rows), at least one 32-entry chunk per split, at
  // most 64 splits; a power of two, so that from kAttnGroupSplits splits on
  // they fill whole workgroups
  const long rows = (long)B * n_q;
  const int chunks = (topk + 31) / 32;
  int ns = 1;
  while (ns < 64 && 2 * ns <= chunks && rows * 2 * ns <= 2048) ns *= 2;
  return ns;
}

size_t attn_workspace_bytes(int B, int n_q, int n_k, int H, int D, int topk) {
  (void)n_k;
  const int parts = attn_nparts(attn_nsplit(B, n_q, topk));
  if (parts <= 1) return 0;
  return round_up((size_t)B * n_q * parts * H * attn_part_stride(D) * 4, 256);
}

}  // namespace dsa

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(dsa_status st) {
  switch (st) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_BAD_PATTERN: return "DSA_ERR_BAD_PATTERN";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

dsa_status dsa_resolve_pattern(int32_t n_layers, const char* pattern, int32_t freq, char* out) {
  if (!out) return fail(DSA_ERR_INVALID_ARGUMENT, "resolve_pattern: out is NULL");
  if (n_layers < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "resolve_pattern: n_layers=%d must be >= 1", n_layers);
  if (freq < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "resolve_pattern: index_topk_freq=%d must be >= 0", freq);
  if (pattern && freq > 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "resolve_pattern: index_topk_pattern and index_topk_freq are alternatives");
  if (pattern) {
    const size_t len = strnlen(pattern, (size_t)n_layers + 1);
    if (len != (size_t)n_layers)
      return fail(DSA_ERR_BAD_PATTERN, "resolve_pattern: pattern length %zu%s != n_layers %d", len,
                  len > (size_t)n_layers ? "+" : "", n_layers);
    for (int l = 0; l < n_layers; ++l)
      if (pattern[l] != 'F' && pattern[l] != 'S')
        return fail(DSA_ERR_BAD_PATTERN, "resolve_pattern: character %d is '%c', not 'F' or 'S'", l, pattern[l]);
    if (pattern[0] != 'F') return fail(DSA_ERR_BAD_PATTERN, "resolve_pattern: the first layer must be 'F'");
    memcpy(out, pattern, (size_t)n_layers);
  } else {
    for (int l = 0; l < n_layers; ++l) out[l] = (freq > 0 && l % freq != 0) ? 'S' : 'F';
  }
  out[n_layers] = '\0';
  return ok();
}

dsa_status dsa_indexer_workspace_size(const dsa_indexer_args* a, size_t* bytes) {
  dsa_status st = check_indexer_shape(a, "indexer_workspace_size");
  if (st != DSA_OK) return st;
  if (!bytes) return fail(DSA_ERR_INVALID_ARGUMENT, "indexer_workspace_size: bytes is NULL");
  *bytes = dsa::indexer_workspace_bytes(a->B, a->n_q, a->n_k, a->topk);
  return ok();
}

dsa_status dsa_attn_workspace_size(const dsa_attn_args* a, size_t* bytes) {
  dsa_status st = check_attn_shape(a, "attn_workspace_size");
  if (st != DSA_OK) return st;
  if (!bytes) return fail(DSA_ERR_INVALID_ARGUMENT, "attn_workspace_size: bytes is NULL");
  *bytes = dsa::attn_workspace_bytes(a->B, a->n_q, a->n_k, a->n_heads, a->head_dim, a->topk);
  return ok();
}

static dsa_status check_stack_shape(const dsa_stack_args* a, const char* what) {
  if (!a) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: args is NULL", what);
  if (a->struct_size != sizeof(dsa_stack_args))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu", what, a->struct_size, sizeof(dsa_stack_args));
  if (a->n_layers < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: n_layers=%d must be >= 1", what, a->n_layers);
  dsa_status st = check_indexer_shape(&a->indexer, what);
  if (st != DSA_OK) return st;
  st = check_attn_shape(&a->attn, what);
  if (st != DSA_OK) return st;
  const dsa_indexer_args& i = a->indexer;
  const dsa_attn_args& t = a->attn;
  if (i.B != t.B || i.n_q != t.n_q || i.n_k != t.n_k || i.q_pos_offset != t.q_pos_offset || i.topk != t.topk)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: indexer and attention shapes disagree (B, n_q, n_k, offset, topk)", what);
  return DSA_OK;
}

static size_t stack_ws(const dsa_stack_args* a) {
  const size_t wi = dsa::indexer_workspace_bytes(a->indexer.B, a->indexer.n_q, a->indexer.n_k, a->indexer.topk);
  const size_t wa = dsa::attn_workspace_bytes(a->attn.B, a->attn.n_q, a->attn.n_k, a->attn.n_heads,
                                              a->attn.head_dim, a->attn.topk);
  return wi > wa ? wi : wa;
}

dsa_status dsa_stack_workspace_size(const dsa_stack_args* a, size_t* bytes) {
  dsa_status st = check_stack_shape(a, "stack_workspace_size");
  if (st != DSA_OK) return st;
  if (!bytes) return fail(DSA_ERR_INVALID_ARGUMENT, "stack_workspace_size: bytes is NULL");
  *bytes = stack_ws(a);
  return ok();
}

dsa_status dsa_indexer_scores_topk(const dsa_indexer_args* a, void* stream) {
  const char* what = "indexer_scores_topk";
  dsa_status st = check_indexer_shape(a, what);
  if (st != DSA_OK) return st;
  st = check_indexer_ptrs(a, a->q, a->k, a->w, a->q_scale, a->k_scale, a->out_idx, what);
  if (st != DSA_OK) return st;
  if ((a->out_scores && !aligned(a->out_scores, 4)) || (a->debug_full_scores && !aligned(a->debug_full_scores, 4)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: misaligned out_scores/debug_full_scores", what);
  const size_t need = dsa::indexer_workspace_bytes(a->B, a->n_q, a->n_k, a->topk);
  st = check_workspace(a->workspace, a->workspace_bytes, need, what);
  if (st != DSA_OK) return st;
  dsa::IndexerParams p = make_indexer_params(a, a->q, a->k, a->w, a->q_scale, a->k_scale, a->out_idx,
                                             a->out_scores, a->debug_full_scores, a->workspace);
  p.ev = a->phase_events;
  st = run_indexer(p, (hipStream_t)stream);
  return st == DSA_OK ? ok() : st;
}

}  // extern "C"

// ---- the no-allocation variant of dsa_indexer_scores_topk
//
// The scratch space lives in this file-scope device array instead of a caller
// workspace. Every GPU the library runs on holds its own copy until the
// process ends. Host code never passes the array's name to a kernel (in host
// code it is only a stand-in for the symbol): the device address of each
// GPU's copy is looked up once per device with hipGetSymbolAddress and kept in
// g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[DSA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of the current device's scratch array, looked up on
// the device's first call.
dsa_status scratch_for_current_device(const char* what, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", what, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", what, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}
}  // namespace

extern "C" {

dsa_status dsa_indexer_scores_topk_static(const dsa_indexer_args* a, void* stream) {
  const char* what = "indexer_scores_topk_static";
  dsa_status st = check_indexer_shape(a, what);
  if (st != DSA_OK) return st;
  st = check_indexer_ptrs(a, a->q, a->k, a->w, a->q_scale, a->k_scale, a->out_idx, what);
  if (st != DSA_OK) return st;
  if ((a->out_scores && !aligned(a->out_scores, 4)) || (a->debug_full_scores && !aligned(a->debug_full_scores, 4)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: misaligned out_scores/debug_full_scores", what);
  if (a->workspace || a->workspace_bytes)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: takes no workspace (workspace must be NULL, workspace_bytes 0)", what);
  const size_t need = dsa::indexer_workspace_bytes(a->B, a->n_q, a->n_k, a->topk);
  if (need > (size_t)DSA_STATIC_SCRATCH_BYTES)
    return fail(DSA_ERR_WORKSPACE, "%s: this shape needs %zu bytes of scratch, the static scratch holds %zu",
                what, need, (size_t)DSA_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_for_current_device(what, &ws);
  if (st != DSA_OK) return st;
  dsa::IndexerParams p = make_indexer_params(a, a->q, a->k, a->w, a->q_scale, a->k_scale, a->out_idx,
                                             a->out_scores, a->debug_full_scores, ws);
  p.ev = a->phase_events;
  st = run_indexer(p, (hipStream_t)stream);
  return st == DSA_OK ? ok() : st;
}

dsa_status dsa_sparse_attn(const dsa_attn_args* a, void* stream) {
  const char* what = "sparse_attn";
  dsa_status st = check_attn_shape(a, what);
  if (st != DSA_OK) return st;
  st = check_attn_ptrs(a->q, a->k, a->v, a->idx, a->out, a->lse, what);
  if (st != DSA_OK) return st;
  const size_t need = dsa::attn_workspace_bytes(a->B, a->n_q, a->n_k, a->n_heads, a->head_dim, a->topk);
  st = check_workspace(a->workspace, a->workspace_bytes, need, what);
  if (st != DSA_OK) return st;
  dsa::AttnParams p = make_attn_params(a, a->q, a->k, a->v, a->idx, a->out, a->lse, a->workspace);
  p.ev = a->phase_events;
  st = run_attn(p, (hipStream_t)stream);
  return st == DSA_OK ? ok() : st;
}

dsa_status dsa_quantize_fp8_rows(const void* x, int64_t rows, int32_t cols, void* out, float* scale, void* stream) {
  const char* what = "quantize_fp8_rows";
  if (rows < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: rows=%lld must be >= 0", what, (long long)rows);
  if (cols < 8 || cols % 8 != 0 || cols > (1 << 24))
    return fail(DSA_ERR_UNSUPPORTED, "%s: cols=%d must be a positive multiple of 8, at most 2^24", what, cols);
  size_t n;
  if (__builtin_mul_overflow((size_t)rows, (size_t)cols, &n) || n > ((size_t)1 << 62))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: rows * cols overflows", what);
  if (rows == 0) return ok();
  if (!x || !out || !scale) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: x, out and scale are required", what);
  if (!aligned(x, 16) || !aligned(out, 8) || !aligned(scale, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: misaligned pointer (x 16 B, out 8 B, scale 4 B)", what);
  const hipError_t e = dsa::launch_quantize_fp8_rows(x, rows, cols, out, scale, (hipStream_t)stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

static dsa_status stack_run(const dsa_stack_args* a, const dsa::PagedKV* kv, const char* pattern, int32_t freq,
                            void* stream, const char* what) {
  dsa_status st = check_stack_shape(a, what);
  if (st != DSA_OK) return st;
  const int n = a->n_layers;
  std::string P((size_t)n + 1, '\0');
  st = dsa_resolve_pattern(n, pattern, freq, &P[0]);
  if (st != DSA_OK) return st;
  if (!a->q_idx || !a->k_idx || !a->w || !a->q || !a->k || !a->v || !a->out || !a->idx_buf)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: per-layer arrays and idx_buf are required", what);
  const bool fp8 = a->indexer.dtype == DSA_FP8_E4M3FN;
  if (fp8 && (!a->q_scale || !a->k_scale))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: fp8 needs q_scale and k_scale arrays", what);
  if (!fp8 && (a->q_scale || a->k_scale))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: q_scale/k_scale arrays must be NULL for bf16", what);
  if (!aligned(a->idx_buf, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: misaligned idx_buf", what);
  for (int l = 0; l < n; ++l) {
    // S layers never read their indexer inputs, but the arrays are validated for
    // every layer so that the same arguments run under any pattern.
    st = check_indexer_ptrs(&a->indexer, a->q_idx[l], a->k_idx[l], a->w[l], fp8 ? a->q_scale[l] : nullptr,
                            fp8 ? a->k_scale[l] : nullptr, a->idx_buf, what);
    if (st != DSA_OK) return fail(st, "%s (layer %d)", dsa_last_error(), l);
    st = check_attn_ptrs(a->q[l], a->k[l], a->v[l], a->idx_buf, a->out[l], a->lse ? a->lse[l] : nullptr, what);
    if (st != DSA_OK) return fail(st, "%s (layer %d)", dsa_last_error(), l);
  }
  st = check_workspace(a->workspace, a->workspace_bytes, stack_ws(a), what);
  if (st != DSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // decode: after the first F layer the histograms and counters are zero and
  // the ragged plan is built, unless the attention partials (at the start of
  // the shared workspace) reach the plan
  const bool decode = a->indexer.n_q == 1;
  const bool keep_prepared =
      decode && dsa::attn_workspace_bytes(a->attn.B, a->attn.n_q, a->attn.n_k, a->attn.n_heads, a->attn.head_dim,
                                          a->attn.topk) <= dsa::indexer_decode_plan_offset(a->indexer.B, a->indexer.n_k,
                                                                                          a->indexer.topk);
  bool prepared = false;
  for (int l = 0; l < n; ++l) {
    if (a->layer_events) {
      const hipError_t e = hipEventRecord((hipEvent_t)a->layer_events[l], s);
      if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipEventRecord: %s", what, hipGetErrorString(e));
    }
    if (P[(size_t)l] == 'F') {
      // F layer: compute fresh indices and overwrite the single cached buffer
      dsa::IndexerParams ip = make_indexer_params(&a->indexer, a->q_idx[l], a->k_idx[l], a->w[l],
                                                  fp8 ? a->q_scale[l] : nullptr, fp8 ? a->k_scale[l] : nullptr,
                                                  a->idx_buf, nullptr, nullptr, a->workspace);
      if (kv) ip.kv = *kv;
      ip.skip_prepare = prepared ? 1 : 0;
      st = run_indexer(ip, s);
      if (st != DSA_OK) return st;
      prepared = keep_prepared;
    }
    // every layer: sparse attention over the cached indices
    dsa::AttnParams ap = make_attn_params(&a->attn, a->q[l], a->k[l], a->v[l], a->idx_buf, a->out[l],
                                          a->lse ? a->lse[l] : nullptr, a->workspace);
    if (kv) ap.kv = *kv;
    st = run_attn(ap, s);
    if (st != DSA_OK) return st;
  }
  if (a->layer_events) {
    const hipError_t e = hipEventRecord((hipEvent_t)a->layer_events[n], s);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipEventRecord: %s", what, hipGetErrorString(e));
  }
  return ok();
}

dsa_status dsa_layer_stack_run(const dsa_stack_args* a, const char* pattern, int32_t freq, void* stream) {
  return stack_run(a, nullptr, pattern, freq, stream, "layer_stack_run");
}

// The stack arguments of chunk [c0, c1) of a chunked prefill: the query rows'
// pointers advanced to row c0 (B = 1, dense rows), the keys cut to the
// chunk's last position, and the caller's per-chunk index buffer. The
// per-layer pointer arrays live in `store` (5 + 2 arrays of n_layers).
static dsa_stack_args chunk_args(const dsa_stack_args* a, int c0, int c1, std::vector<const void*>& store) {
  const int n = a->n_layers;
  const dsa_indexer_args& ix = a->indexer;
  const dsa_attn_args& at = a->attn;
  const bool fp8 = ix.dtype == DSA_FP8_E4M3FN;
  const size_t qi_row = (size_t)ix.n_heads * ix.head_dim * (fp8 ? 1 : 2);
  const size_t q_row = (size_t)at.n_heads * at.head_dim * 2;
  store.assign((size_t)7 * n, nullptr);
  const void** qi = &store[0];
  const void** w = &store[(size_t)n];
  const void** qs = &store[(size_t)2 * n];
  const void** q = &store[(size_t)3 * n];
  const void** out = &store[(size_t)4 * n];
  const void** lse = &store[(size_t)5 * n];
  for (int l = 0; l < n; ++l) {
    qi[l] = a->q_idx[l] ? (const char*)a->q_idx[l] + (size_t)c0 * qi_row : nullptr;
    w[l] = a->w[l] ? a->w[l] + (size_t)c0 * ix.n_heads : nullptr;
    if (a->q_scale) qs[l] = a->q_scale[l] ? a->q_scale[l] + c0 : nullptr;
    q[l] = a->q[l] ? (const char*)a->q[l] + (size_t)c0 * q_row : nullptr;
    out[l] = a->out[l] ? (char*)a->out[l] + (size_t)c0 * q_row : nullptr;
    if (a->lse) lse[l] = a->lse[l] ? a->lse[l] + (size_t)c0 * at.n_heads : nullptr;
  }
  dsa_stack_args c = *a;
  c.indexer.n_q = c.attn.n_q = c1 - c0;
  c.indexer.q_pos_offset = c.attn.q_pos_offset = ix.q_pos_offset + c0;
  c.indexer.n_k = c.attn.n_k = ix.q_pos_offset + c1;
  c.q_idx = qi;
  c.w = (const float* const*)w;
  c.q_scale = a->q_scale ? (const float* const*)qs : nullptr;
  c.q = q;
  c.out = (void* const*)out;
  c.lse = a->lse ? (float* const*)lse : nullptr;
  c.layer_events = nullptr;
  return c;
}

static dsa_status check_chunked(const dsa_stack_args* a, int32_t chunk_rows, const char* what) {
  dsa_status st = check_stack_shape(a, what);
  if (st != DSA_OK) return st;
  if (a->indexer.B != 1)
    return fail(DSA_ERR_UNSUPPORTED, "%s: chunked prefill takes one sequence (B = 1), got B = %d", what, a->indexer.B);
  if (chunk_rows < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: chunk_rows=%d must be >= 1", what, chunk_rows);
  if (a->layer_events) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: layer_events must be NULL (per-layer events do not span chunks)", what);
  return DSA_OK;
}

// Workspace of the largest chunk shape: a full chunk and the ragged last one
// (the attention split, hence its partials, depends on the row count; a
// one-row chunk takes the decode path).
static size_t chunked_ws(const dsa_stack_args* a, int32_t chunk_rows) {
  const int n_q = a->indexer.n_q;
  const int full = std::min(chunk_rows, n_q);
  const int last = n_q % full;
  size_t need = 0;
  for (int rows : {full, last}) {
    if (rows < 1) continue;
    dsa_stack_args c = *a;
    c.indexer.n_q = c.attn.n_q = rows;
    c.indexer.q_pos_offset = c.attn.q_pos_offset = a->indexer.n_k - rows;  // the largest key count
    need = std::max(need, stack_ws(&c));
  }
  return need;
}

dsa_status dsa_chunked_stack_workspace_size(const dsa_stack_args* a, int32_t chunk_rows, size_t* bytes) {
  const char* what = "chunked_stack_workspace_size";
  dsa_status st = check_chunked(a, chunk_rows, what);
  if (st != DSA_OK) return st;
  if (!bytes) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", what);
  *bytes = chunked_ws(a, chunk_rows);
  return ok();
}

dsa_status dsa_layer_stack_run_chunked(const dsa_stack_args* a, int32_t chunk_rows, const char* pattern, int32_t freq,
                                       void* stream) {
  const char* what = "layer_stack_run_chunked";
  dsa_status st = check_chunked(a, chunk_rows, what);
  if (st != DSA_OK) return st;
  const int n_q = a->indexer.n_q;
  std::string P((size_t)a->n_layers + 1, '\0');
  st = dsa_resolve_pattern(a->n_layers, pattern, freq, &P[0]);
  if (st != DSA_OK) return st;
  if (!a->q_idx || !a->k_idx || !a->w || !a->q || !a->k || !a->v || !a->out || !a->idx_buf)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: per-layer arrays and idx_buf are required", what);
  st = check_workspace(a->workspace, a->workspace_bytes, chunked_ws(a, chunk_rows), what);
  if (st != DSA_OK) return st;
  // every chunk's arguments are validated before the first one is enqueued
  std::vector<const void*> store;
  for (int c0 = 0; c0 < n_q; c0 += chunk_rows) {
    const int c1 = std::min(n_q, c0 + chunk_rows);
    dsa_stack_args c = chunk_args(a, c0, c1, store);
    st = check_stack_shape(&c, what);
    if (st != DSA_OK) return fail(st, "%s (chunk at row %d)", dsa_last_error(), c0);
    if (c0 > 0) continue;
    // pointers and alignment are the same for every chunk up to the row offsets
    const bool fp8 = c.indexer.dtype == DSA_FP8_E4M3FN;
    for (int l = 0; l < c.n_layers; ++l) {
      st = check_indexer_ptrs(&c.indexer, c.q_idx[l], c.k_idx[l], c.w[l], fp8 ? c.q_scale[l] : nullptr,
                              fp8 ? c.k_scale[l] : nullptr, c.idx_buf, what);
      if (st != DSA_OK) return fail(st, "%s (layer %d)", dsa_last_error(), l);
      st = check_attn_ptrs(c.q[l], c.k[l], c.v[l], c.idx_buf, c.out[l], c.lse ? c.lse[l] : nullptr, what);
      if (st != DSA_OK) return fail(st, "%s (layer %d)", dsa_last_error(), l);
    }
  }
  for (int c0 = 0; c0 < n_q; c0 += chunk_rows) {
    const int c1 = std::min(n_q, c0 + chunk_rows);
    dsa_stack_args c = chunk_args(a, c0, c1, store);
    st = stack_run(&c, nullptr, P.c_str(), 0, stream, what);
    if (st != DSA_OK) return fail(st, "%s (chunk at row %d)", dsa_last_error(), c0);
  }
  return ok();
}

// Validates the paged layout for decode shapes (n_q == 1, n_k == max_seq_len)
// and fills the kernels' view of it.
static dsa_status check_paged(const dsa_paged_kv* kv, int B, int n_q, int n_k, int64_t row_bytes, const char* what,
                              dsa::PagedKV* out) {
  if (!kv) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: kv is NULL", what);
  if (kv->struct_size != sizeof(dsa_paged_kv))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: kv struct_size %u != %zu", what, kv->struct_size, sizeof(dsa_paged_kv));
  if (n_q != 1) return fail(DSA_ERR_UNSUPPORTED, "%s: paged calls are decode only (n_q must be 1, got %d)", what, n_q);
  if (kv->max_seq_len < 1 || n_k != kv->max_seq_len)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: n_k (%d) must equal kv->max_seq_len (%d) >= 1", what, n_k,
                kv->max_seq_len);
  if (kv->page_size < 32 || kv->page_size % 32 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "%s: page_size=%d must be a positive multiple of 32", what, kv->page_size);
  if (kv->max_pages < 1 || kv->num_pages < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: max_pages and num_pages must be >= 1", what);
  if ((int64_t)kv->max_pages * kv->page_size < kv->max_seq_len)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: max_pages * page_size < max_seq_len", what);
  int64_t n;
  if ((int64_t)kv->num_pages * kv->page_size > INT32_MAX ||
      !count4(kv->num_pages, kv->page_size, row_bytes, 1, &n) || !count4(B, kv->max_pages, 1, 1, &n))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: pool or block table sizes overflow", what);
  if (!kv->seq_lens || !kv->block_table || !aligned(kv->seq_lens, 4) || !aligned(kv->block_table, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: seq_lens and block_table are required (4-byte aligned)", what);
  out->seq_lens = kv->seq_lens;
  out->block_table = kv->block_table;
  out->page_size = kv->page_size;
  out->max_pages = kv->max_pages;
  out->num_pages = kv->num_pages;
  return DSA_OK;
}

dsa_status dsa_paged_indexer_topk(const dsa_indexer_args* a, const dsa_paged_kv* kv, void* stream) {
  const char* what = "paged_indexer_topk";
  dsa_status st = check_indexer_shape(a, what);
  if (st != DSA_OK) return st;
  dsa::PagedKV pk;
  st = check_paged(kv, a->B, a->n_q, a->n_k, (int64_t)a->head_dim * (a->dtype == DSA_FP8_E4M3FN ? 1 : 2), what, &pk);
  if (st != DSA_OK) return st;
  st = check_indexer_ptrs(a, a->q, a->k, a->w, a->q_scale, a->k_scale, a->out_idx, what);
  if (st != DSA_OK) return st;
  if ((a->out_scores && !aligned(a->out_scores, 4)) || (a->debug_full_scores && !aligned(a->debug_full_scores, 4)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: misaligned out_scores/debug_full_scores", what);
  const size_t need = dsa::indexer_workspace_bytes(a->B, a->n_q, a->n_k, a->topk);
  st = check_workspace(a->workspace, a->workspace_bytes, need, what);
  if (st != DSA_OK) return st;
  dsa::IndexerParams p = make_indexer_params(a, a->q, a->k, a->w, a->q_scale, a->k_scale, a->out_idx,
                                             a->out_scores, a->debug_full_scores, a->workspace);
  p.kv = pk;
  p.ev = a->phase_events;
  st = run_indexer(p, (hipStream_t)stream);
  return st == DSA_OK ? ok() : st;
}

dsa_status dsa_paged_sparse_attn(const dsa_attn_args* a, const dsa_paged_kv* kv, void* stream) {
  const char* what = "paged_sparse_attn";
  dsa_status st = check_attn_shape(a, what);
  if (st != DSA_OK) return st;
  dsa::PagedKV pk;
  st = check_paged(kv, a->B, a->n_q, a->n_k, (int64_t)a->head_dim * 2, what, &pk);
  if (st != DSA_OK) return st;
  st = check_attn_ptrs(a->q, a->k, a->v, a->idx, a->out, a->lse, what);
  if (st != DSA_OK) return st;
  const size_t need = dsa::attn_workspace_bytes(a->B, a->n_q, a->n_k, a->n_heads, a->head_dim, a->topk);
  st = check_workspace(a->workspace, a->workspace_bytes, need, what);
  if (st != DSA_OK) return st;
  dsa::AttnParams p = make_attn_params(a, a->q, a->k, a->v, a->idx, a->out, a->lse, a->workspace);
  p.kv = pk;
  p.ev = a->phase_events;
  st = run_attn(p, (hipStream_t)stream);
  return st == DSA_OK ? ok() : st;
}

dsa_status dsa_paged_layer_stack_run(const dsa_stack_args* a, const dsa_paged_kv* kv, const char* pattern,
                                     int32_t freq, void* stream) {
  const char* what = "paged_layer_stack_run";
  dsa_status st = check_stack_shape(a, what);
  if (st != DSA_OK) return st;
  dsa::PagedKV pk;
  const int64_t rb = std::max<int64_t>((int64_t)a->indexer.head_dim * 2, (int64_t)a->attn.head_dim * 2);
  st = check_paged(kv, a->indexer.B, a->indexer.n_q, a->indexer.n_k, rb, what, &pk);
  if (st != DSA_OK) return st;
  return stack_run(a, &pk, pattern, freq, stream, what);
}

dsa_status dsa_paged_append_rows(const void* src, int32_t B, int32_t row_bytes, void* pool, const dsa_paged_kv* kv,
                                 void* stream) {
  const char* what = "paged_append_rows";
  if (B < 1 || B > kMaxB) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: B=%d out of 1..%d", what, B, kMaxB);
  if (row_bytes < 4 || row_bytes % 4 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "%s: row_bytes=%d must be a positive multiple of 4", what, row_bytes);
  dsa::PagedKV pk;
  dsa_status st = check_paged(kv, B, 1, kv ? kv->max_seq_len : 0, row_bytes, what, &pk);
  if (st != DSA_OK) return st;
  if (!src || !pool || !aligned(src, 4) || !aligned(pool, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: src and pool are required (4-byte aligned)", what);
  const hipError_t e = dsa::launch_paged_append_rows(src, B, row_bytes, pool, pk, kv->max_seq_len, (hipStream_t)stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

dsa_status dsa_topk_overlap(const int32_t* idx, int32_t n_layers, int32_t rows, int32_t topk, int32_t n_k,
                            int64_t* inter, void* stream) {
  const char* what = "topk_overlap";
  if (n_layers < 1 || n_layers > kMaxOverlapLayers)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: n_layers=%d out of 1..%d", what, n_layers, kMaxOverlapLayers);
  if (rows < 1 || topk < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: rows=%d topk=%d must be >= 1", what, rows, topk);
  if (n_k < 1 || n_k > kMaxOverlapKeys)
    return fail(DSA_ERR_UNSUPPORTED, "%s: n_k=%d out of 1..%d (the bitmap lives in LDS)", what, n_k, kMaxOverlapKeys);
  int64_t n;
  if (!count4(n_layers, rows, topk, 4, &n)) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: sizes overflow int64", what);
  if (!idx || !inter || !aligned(idx, 4) || !aligned(inter, 8))
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: idx (4-byte aligned) and inter (8-byte aligned) are required", what);
  const hipError_t e = dsa::launch_topk_overlap(idx, n_layers, rows, topk, n_k, inter, (hipStream_t)stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

dsa_status dsa_similarity_pattern(int32_t n_layers, const int64_t* inter, int32_t n_full, char* out) {
  const char* what = "similarity_pattern";
  if (!inter || !out) return fail(DSA_ERR_INVALID_ARGUMENT, "%s: inter and out are required", what);
  if (n_layers < 1 || n_layers > kMaxOverlapLayers)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: n_layers=%d out of 1..%d", what, n_layers, kMaxOverlapLayers);
  if (n_full < 1 || n_full > n_layers)
    return fail(DSA_ERR_INVALID_ARGUMENT, "%s: n_full=%d out of 1..%d", what, n_full, n_layers);
  const int L = n_layers;
  for (int64_t i = 0; i < (int64_t)L * L; ++i)
    if (inter[i] < 0 || inter[i] > ((int64_t)1 << 52))
      return fail(DSA_ERR_INVALID_ARGUMENT, "%s: inter[%lld] = %lld outside 0..2^52", what, (long long)i,
                  (long long)inter[i]);
  // seg(i, e) = sum_{i < l < e} inter[i][l]: prefix sums of each row
  std::vector<int64_t> pre((size_t)L * (L + 1), 0);
  for (int i = 0; i < L; ++i)
    for (int l = 0; l < L; ++l) pre[(size_t)i * (L + 1) + l + 1] = pre[(size_t)i * (L + 1) + l] + inter[(size_t)i * L + l];
  auto seg = [&](int i, int e) { return pre[(size_t)i * (L + 1) + e] - pre[(size_t)i * (L + 1) + i + 1]; };
  // V[i][j]: best shared selections of layers i..L-1 with layer i F and j F
  // layers in i..L-1 (-1: impossible)
  const int J = n_full;
  std::vector<int64_t> V((size_t)(L + 1) * (J + 1), -1);
  auto at = [&](int i, int j) -> int64_t& { return V[(size_t)i * (J + 1) + j]; };
  for (int i = L - 1; i >= 0; --i) {
    at(i, 1) = seg(i, L);
    for (int j = 2; j <= J && j <= L - i; ++j) {
      int64_t best = -1;
      for (int e = i + 1; e <= L - j + 1; ++e)
        if (at(e, j - 1) >= 0) best = std::max(best, seg(i, e) + at(e, j - 1));
      at(i, j) = best;
    }
  }
  // F layers front to back: the smallest next F layer that keeps the optimum
  for (int l = 0; l < L; ++l) out[l] = 'S';
  out[L] = '\0';
  out[0] = 'F';
  for (int i = 0, j = J; j > 1; --j) {
    const int64_t target = at(i, j);
    int e = i + 1;
    while (!(at(e, j - 1) >= 0 && seg(i, e) + at(e, j - 1) == target)) ++e;
    out[e] = 'F';
    i = e;
  }
  return ok();
}

}  // extern "C"
