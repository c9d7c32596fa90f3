// Host side of the C ABI declared in include/lca.h: argument validation, the
// grouping plan, workspace sizing, thread-local error text and kernel
// dispatch on the caller's stream. No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "lca.h"
#include "lca_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return LCA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool valid_dtype(int32_t d) { return d == LCA_BF16 || d == LCA_F32; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool mult8(int64_t s) { return s % 8 == 0; }

// A latent tensor used for 16-byte row loads/stores.
int check_latent(const lca_latent_t* t, const char* name, bool need_c, bool need_kr) {
  if (t == nullptr) return fail(LCA_ERR_INVALID_ARG, "%s is null", name);
  if (!valid_dtype(t->dtype)) return fail(LCA_ERR_INVALID_ARG, "%s->dtype %d is not LCA_BF16/LCA_F32", name, t->dtype);
  if (need_c && (t->c == nullptr || !aligned16(t->c)))
    return fail(LCA_ERR_INVALID_ARG, "%s->c must be a non-null 16-byte aligned pointer", name);
  if (need_kr && (t->kr == nullptr || !aligned16(t->kr)))
    return fail(LCA_ERR_INVALID_ARG, "%s->kr must be a non-null 16-byte aligned pointer", name);
  if (!mult8(t->c_seq_stride) || !mult8(t->c_tok_stride) || !mult8(t->kr_seq_stride) ||
      !mult8(t->kr_tok_stride) || t->c_tok_stride < 0 || t->kr_tok_stride < 0 ||
      t->c_seq_stride < 0 || t->kr_seq_stride < 0)
    return fail(LCA_ERR_INVALID_ARG, "%s strides must be non-negative multiples of 8 elements", name);
  return LCA_OK;
}

int check_scale(float s) {
  if (!std::isfinite(s) || s < 0.f) return fail(LCA_ERR_INVALID_ARG, "sm_scale must be finite and >= 0");
  return LCA_OK;
}

}  // namespace

extern "C" {

int lca_version(void) { return LCA_VERSION; }

const char* lca_last_error(void) { return g_err.c_str(); }

int lca_plan(int64_t L, int64_t w, int32_t g, lca_plan_t* out) {
  if (out == nullptr) return fail(LCA_ERR_INVALID_ARG, "out is null");
  if (L < 0 || w < 0 || g < 1) return fail(LCA_ERR_INVALID_ARG, "need L >= 0, w >= 0, g >= 1");
  const int64_t m = L > w ? (L - w) / g : 0;
  out->m = m;
  out->raw_begin = m * g;
  out->raw_end = L;
  out->n_entries = m + (L - m * g);
  return ok();
}

size_t lca_condense_workspace_size(int32_t B, int64_t n_groups, int64_t q_row_step) {
  if (B < 1 || n_groups < 0) return 0;
  // per-group summary queries, or one per sequence plus its partial sums
  const int64_t nq = q_row_step != 0 ? n_groups : (n_groups > 0 ? 1 + lca::QBAR_PARTS : 0);
  return (size_t)B * (size_t)nq * LCA_D_ROW * sizeof(float);
}

int lca_condense(const lca_latent_t* cache, int32_t B, int32_t g, int64_t group_begin,
                 int64_t n_groups, const void* q, int32_t q_dtype, int64_t q_seq_stride,
                 int64_t q_tok_stride, int64_t T, int32_t H, int64_t q_row0,
                 int64_t q_row_step, float sm_scale, const lca_latent_t* reps,
                 int32_t* anchor_idx, int64_t anchor_seq_stride, float* alpha,
                 int64_t alpha_seq_stride, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  return lca_condense_mode(cache, B, g, group_begin, n_groups, q, q_dtype, q_seq_stride, q_tok_stride, T,
                           H, q_row0, q_row_step, sm_scale, reps, anchor_idx, anchor_seq_stride, alpha,
                           alpha_seq_stride, workspace, workspace_bytes, LCA_MODE_LCA, stream);
}

int lca_condense_mode(const lca_latent_t* cache, int32_t B, int32_t g, int64_t group_begin,
                      int64_t n_groups, const void* q, int32_t q_dtype, int64_t q_seq_stride,
                      int64_t q_tok_stride, int64_t T, int32_t H, int64_t q_row0,
                      int64_t q_row_step, float sm_scale, const lca_latent_t* reps,
                      int32_t* anchor_idx, int64_t anchor_seq_stride, float* alpha,
                      int64_t alpha_seq_stride, void* workspace, size_t workspace_bytes,
                      int32_t mode, hipStream_t stream) {
  int rc;
  if (mode != LCA_MODE_LCA && mode != LCA_MODE_POOL_ROPE && mode != LCA_MODE_ANCHOR)
    return fail(LCA_ERR_INVALID_ARG, "mode %d is not an lca_mode_t", mode);
  if ((rc = check_latent(cache, "cache", true, true)) != LCA_OK) return rc;
  if ((rc = check_latent(reps, "reps", true, true)) != LCA_OK) return rc;
  if (B < 1 || B > 65535) return fail(LCA_ERR_INVALID_ARG, "B must be in [1, 65535]");
  if (g < 1 || g > LCA_MAX_G || (g & (g - 1)) != 0)
    return fail(LCA_ERR_UNSUPPORTED, "g = %d: supported group sizes are powers of two up to %d", g, LCA_MAX_G);
  if (H < 1) return fail(LCA_ERR_INVALID_ARG, "H must be >= 1");
  if (group_begin < 0 || n_groups < 0) return fail(LCA_ERR_INVALID_ARG, "group_begin and n_groups must be >= 0");
  if (n_groups > ((int64_t)1 << 32)) return fail(LCA_ERR_UNSUPPORTED, "too many groups in one call");
  if (q == nullptr || !aligned16(q)) return fail(LCA_ERR_INVALID_ARG, "q must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (!mult8(q_seq_stride) || !mult8(q_tok_stride) || q_seq_stride < 0 || q_tok_stride < 0)
    return fail(LCA_ERR_INVALID_ARG, "q strides must be non-negative multiples of 8 elements");
  if (anchor_idx == nullptr) return fail(LCA_ERR_INVALID_ARG, "anchor_idx is null");
  if (anchor_seq_stride < 0 || alpha_seq_stride < 0) return fail(LCA_ERR_INVALID_ARG, "negative output stride");
  if ((rc = check_scale(sm_scale)) != LCA_OK) return rc;
  if (q_row0 < 0 || q_row_step < 0) return fail(LCA_ERR_INVALID_ARG, "q_row0 and q_row_step must be >= 0");
  if (n_groups == 0) return ok();
  const int64_t last_row = q_row0 + (n_groups - 1) * q_row_step + g - 1;
  if (last_row >= T) return fail(LCA_ERR_INVALID_ARG, "summary-query rows reach row %lld but T = %lld", (long long)last_row, (long long)T);
  if (q_row_step != 0 && n_groups > 0x7fffffff) return fail(LCA_ERR_UNSUPPORTED, "too many summary queries");
  const size_t need = lca_condense_workspace_size(B, n_groups, q_row_step);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return fail(LCA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  return hip_status(lca::launch_condense(*cache, B, g, group_begin, n_groups, q, q_dtype, q_seq_stride,
                                         q_tok_stride, H, q_row0, q_row_step, sm_scale, *reps,
                                         anchor_idx, anchor_seq_stride, alpha, alpha_seq_stride,
                                         static_cast<float*>(workspace), mode, stream),
                    "lca_condense launch");
}

int lca_condense_paged(const lca_paged_t* cache, int32_t B, int32_t g, const int32_t* seq_group_begin,
                       const int32_t* seq_n_groups, int64_t max_groups, const void* q, int32_t q_dtype,
                       int64_t q_seq_stride, int64_t q_tok_stride, int64_t T, int32_t H, int64_t q_row0,
                       int64_t q_row_step, float sm_scale, const lca_latent_t* reps, int32_t* anchor_idx,
                       int64_t anchor_seq_stride, float* alpha, int64_t alpha_seq_stride,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc;
  if (cache == nullptr || cache->pages == nullptr || !aligned16(cache->pages))
    return fail(LCA_ERR_INVALID_ARG, "cache pages must be a non-null 16-byte aligned pointer");
  if (cache->row_stride < LCA_D_ROW || !mult8(cache->row_stride))
    return fail(LCA_ERR_INVALID_ARG, "cache row_stride must be >= 576 and a multiple of 8");
  if (cache->block_table == nullptr || cache->table_stride < 1)
    return fail(LCA_ERR_INVALID_ARG, "block_table must be non-null with table_stride >= 1");
  if (B < 1 || B > 65535) return fail(LCA_ERR_INVALID_ARG, "B must be in [1, 65535]");
  if (g < 1 || g > LCA_MAX_G || (g & (g - 1)) != 0)
    return fail(LCA_ERR_UNSUPPORTED, "g = %d: supported group sizes are powers of two up to %d", g, LCA_MAX_G);
  if (cache->page_rows < 1 || cache->page_rows % g != 0)
    return fail(LCA_ERR_UNSUPPORTED, "page_rows = %d must be a positive multiple of g = %d", cache->page_rows, g);
  if (seq_group_begin == nullptr || seq_n_groups == nullptr)
    return fail(LCA_ERR_INVALID_ARG, "seq_group_begin and seq_n_groups must be non-null device arrays");
  if (max_groups < 0 || max_groups > ((int64_t)1 << 31)) return fail(LCA_ERR_INVALID_ARG, "max_groups must be in [0, 2^31]");
  if (H < 1) return fail(LCA_ERR_INVALID_ARG, "H must be >= 1");
  if (q == nullptr || !aligned16(q)) return fail(LCA_ERR_INVALID_ARG, "q must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (!mult8(q_seq_stride) || !mult8(q_tok_stride) || q_seq_stride < 0 || q_tok_stride < 0)
    return fail(LCA_ERR_INVALID_ARG, "q strides must be non-negative multiples of 8 elements");
  if (q_row0 < 0 || q_row_step < 0) return fail(LCA_ERR_INVALID_ARG, "q_row0 and q_row_step must be >= 0");
  if (q_row_step != 0 && max_groups > 0x7fffffff) return fail(LCA_ERR_UNSUPPORTED, "too many summary queries");
  {
    const int64_t last_row = q_row0 + (max_groups > 0 ? max_groups - 1 : 0) * q_row_step + g - 1;
    if (last_row >= T)
      return fail(LCA_ERR_INVALID_ARG, "summary-query rows reach row %lld but T = %lld", (long long)last_row, (long long)T);
  }
  if ((rc = check_latent(reps, "reps", true, true)) != LCA_OK) return rc;
  if (reps->dtype != LCA_BF16 || static_cast<const char*>(reps->kr) != static_cast<const char*>(reps->c) + 2 * LCA_D_C ||
      reps->kr_tok_stride != reps->c_tok_stride || reps->kr_seq_stride != reps->c_seq_stride)
    return fail(LCA_ERR_UNSUPPORTED, "paged condensation writes packed bf16 representatives (k_R right after c_KV)");
  if (anchor_idx == nullptr) return fail(LCA_ERR_INVALID_ARG, "anchor_idx is null");
  if (anchor_seq_stride < 0 || alpha_seq_stride < 0) return fail(LCA_ERR_INVALID_ARG, "negative output stride");
  if ((rc = check_scale(sm_scale)) != LCA_OK) return rc;
  if (max_groups == 0) return ok();
  const size_t need = lca_condense_workspace_size(B, max_groups, q_row_step);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return fail(LCA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  return hip_status(lca::launch_condense_paged(*cache, B, g, seq_group_begin, seq_n_groups, max_groups, q, q_dtype,
                                               q_seq_stride, q_tok_stride, H, q_row0, q_row_step, sm_scale, *reps, anchor_idx,
                                               anchor_seq_stride, alpha, alpha_seq_stride,
                                               static_cast<float*>(workspace), stream),
                    "lca_condense_paged launch");
}

}  // extern "C"

namespace {
// Arguments of the step condensation (lca_condense_step, and the step part of
// mla_latent_attn_decode_paged_up_step) other than the query buffer.
int check_step(const lca_paged_t* cache, int32_t B, int64_t w, int32_t g, int32_t H, const void* q_ring,
               int64_t q_ring_seq_stride, const lca_latent_t* reps, const int32_t* anchor_idx,
               int64_t anchor_seq_stride, const int32_t* seq_m, const int32_t* seq_raw_begin,
               const int32_t* seq_raw_end) {
  int rc;
  if (cache == nullptr || cache->pages == nullptr || !aligned16(cache->pages))
    return fail(LCA_ERR_INVALID_ARG, "cache pages must be a non-null 16-byte aligned pointer");
  if (cache->row_stride < LCA_D_ROW || !mult8(cache->row_stride))
    return fail(LCA_ERR_INVALID_ARG, "cache row_stride must be >= 576 and a multiple of 8");
  if (cache->block_table == nullptr || cache->table_stride < 1)
    return fail(LCA_ERR_INVALID_ARG, "block_table must be non-null with table_stride >= 1");
  if (B < 1 || B > 65535) return fail(LCA_ERR_INVALID_ARG, "B must be in [1, 65535]");
  if (w < 0) return fail(LCA_ERR_INVALID_ARG, "w must be >= 0");
  if (g < 1 || g > LCA_MAX_G || (g & (g - 1)) != 0)
    return fail(LCA_ERR_UNSUPPORTED, "g = %d: supported group sizes are powers of two up to %d", g, LCA_MAX_G);
  if (cache->page_rows < 1 || cache->page_rows % g != 0)
    return fail(LCA_ERR_UNSUPPORTED, "page_rows = %d must be a positive multiple of g = %d", cache->page_rows, g);
  if (H < 1 || H > 1024) return fail(LCA_ERR_INVALID_ARG, "H must be in [1, 1024]");
  if (q_ring == nullptr || !aligned16(q_ring))
    return fail(LCA_ERR_INVALID_ARG, "q_ring must be a non-null 16-byte aligned pointer");
  if (!mult8(q_ring_seq_stride) || q_ring_seq_stride < (int64_t)g * H * LCA_D_ROW)
    return fail(LCA_ERR_INVALID_ARG, "q_ring_seq_stride must be a multiple of 8 and >= g * H * 576 = %lld",
                (long long)g * H * LCA_D_ROW);
  if ((rc = check_latent(reps, "reps", true, true)) != LCA_OK) return rc;
  if (reps->dtype != LCA_BF16 || static_cast<const char*>(reps->kr) != static_cast<const char*>(reps->c) + 2 * LCA_D_C ||
      reps->kr_tok_stride != reps->c_tok_stride || reps->kr_seq_stride != reps->c_seq_stride)
    return fail(LCA_ERR_UNSUPPORTED, "the step condensation writes packed bf16 representatives (k_R right after c_KV)");
  if (anchor_idx == nullptr) return fail(LCA_ERR_INVALID_ARG, "anchor_idx is null");
  if (anchor_seq_stride < 0) return fail(LCA_ERR_INVALID_ARG, "negative anchor_seq_stride");
  if (seq_m == nullptr || seq_raw_begin == nullptr || seq_raw_end == nullptr)
    return fail(LCA_ERR_INVALID_ARG, "seq_m, seq_raw_begin and seq_raw_end must be non-null device arrays");
  return LCA_OK;
}
}  // namespace

extern "C" {

int lca_condense_step(const lca_paged_t* cache, int32_t B, int64_t w, int32_t g, const void* q, int32_t q_dtype,
                      int64_t q_seq_stride, int32_t H, void* q_ring, int64_t q_ring_seq_stride, float sm_scale,
                      const lca_latent_t* reps, int32_t* anchor_idx, int64_t anchor_seq_stride, int32_t* seq_m,
                      int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos, int64_t* dst_row,
                      hipStream_t stream) {
  int rc;
  if ((rc = check_step(cache, B, w, g, H, q_ring, q_ring_seq_stride, reps, anchor_idx, anchor_seq_stride, seq_m,
                       seq_raw_begin, seq_raw_end)) != LCA_OK)
    return rc;
  if (q == nullptr || !aligned16(q)) return fail(LCA_ERR_INVALID_ARG, "q must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (!mult8(q_seq_stride) || q_seq_stride < 0)
    return fail(LCA_ERR_INVALID_ARG, "q_seq_stride must be a non-negative multiple of 8 elements");
  if ((rc = check_scale(sm_scale)) != LCA_OK) return rc;
  return hip_status(lca::launch_condense_step(*cache, B, w, g, q, q_dtype, q_seq_stride, H, q_ring, q_ring_seq_stride,
                                              sm_scale, *reps, anchor_idx, anchor_seq_stride, seq_m, seq_raw_begin,
                                              seq_raw_end, pos, dst_row, stream),
                    "lca_condense_step launch");
}

size_t mla_latent_attn_decode_workspace_size(int32_t B, int32_t H, int64_t max_entries) {
  if (B < 1 || !lca::heads_supported(H) || max_entries < 1) return 0;
  const lca::DecodeSplit sp = lca::decode_split(B, lca::head_blocks(H), max_entries);
  return lca::decode_workspace_bytes(B, lca::head_blocks(H), sp.S);
}

int mla_latent_attn_decode(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                           int32_t H, const lca_latent_t* reps, int64_t m,
                           const lca_latent_t* raw, int64_t raw_begin, int64_t raw_end,
                           float sm_scale, float* o_latent, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  int rc;
  if (q == nullptr || !aligned16(q)) return fail(LCA_ERR_INVALID_ARG, "q must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (!mult8(q_seq_stride) || q_seq_stride < 0) return fail(LCA_ERR_INVALID_ARG, "q_seq_stride must be a non-negative multiple of 8");
  if (B < 1 || B > 65535) return fail(LCA_ERR_INVALID_ARG, "B must be in [1, 65535]");
  if (!lca::heads_supported(H) || lca::head_blocks(H) > 65535)
    return fail(LCA_ERR_UNSUPPORTED, "H = %d: the head count must be a multiple of 16 or divide 16", H);
  if (m < 0 || raw_begin < 0 || raw_end < raw_begin) return fail(LCA_ERR_INVALID_ARG, "need m >= 0 and 0 <= raw_begin <= raw_end");
  const int64_t n = m + (raw_end - raw_begin);
  if (n < 1) return fail(LCA_ERR_INVALID_ARG, "nothing to attend: m + raw_end - raw_begin must be >= 1");
  if (m > 0 && (rc = check_latent(reps, "reps", true, true)) != LCA_OK) return rc;
  if (raw_end > raw_begin && (rc = check_latent(raw, "raw", true, true)) != LCA_OK) return rc;
  if (m > 0 && raw_end > raw_begin && reps->dtype != raw->dtype)
    return fail(LCA_ERR_UNSUPPORTED, "reps and raw must share one dtype");
  if ((rc = check_scale(sm_scale)) != LCA_OK) return rc;
  if (o_latent == nullptr || !aligned16(o_latent)) return fail(LCA_ERR_INVALID_ARG, "o_latent must be a non-null 16-byte aligned pointer");
  const lca::DecodeSplit sp = lca::decode_split(B, lca::head_blocks(H), n);
  const size_t need = lca::decode_workspace_bytes(B, lca::head_blocks(H), sp.S);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  const lca_latent_t none = {nullptr, nullptr, 0, 0, 0, 0, m > 0 ? reps->dtype : raw->dtype};
  const lca_latent_t& rp = m > 0 ? *reps : none;
  const lca_latent_t& rw = raw_end > raw_begin ? *raw : none;
  return hip_status(lca::launch_decode(q, q_dtype, q_seq_stride, B, H, rp, m, rw, raw_begin, raw_end,
                                       sm_scale, o_latent, lse, workspace, stream),
                    "mla_latent_attn_decode launch");
}

}  // extern "C"

namespace {
// Arguments of mla_latent_attn_decode_paged / _paged_up shared by both;
// on success *need receives the bytes of split-K partials.
int check_decode_paged(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B, int32_t H,
                       const lca_latent_t* reps, const int32_t* seq_m, const lca_paged_t* cache,
                       const int32_t* seq_raw_begin, const int32_t* seq_raw_end, int64_t max_entries,
                       float sm_scale, float* o_latent, size_t* need) {
  int rc;
  if (q == nullptr || !aligned16(q)) return fail(LCA_ERR_INVALID_ARG, "q must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (!mult8(q_seq_stride) || q_seq_stride < 0) return fail(LCA_ERR_INVALID_ARG, "q_seq_stride must be a non-negative multiple of 8");
  if (B < 1 || B > 65535) return fail(LCA_ERR_INVALID_ARG, "B must be in [1, 65535]");
  if (!lca::heads_supported(H) || lca::head_blocks(H) > 65535)
    return fail(LCA_ERR_UNSUPPORTED, "H = %d: the head count must be a multiple of 16 or divide 16", H);
  if (cache == nullptr || cache->pages == nullptr || !aligned16(cache->pages))
    return fail(LCA_ERR_INVALID_ARG, "cache pages must be a non-null 16-byte aligned pointer");
  if (cache->row_stride < LCA_D_ROW || !mult8(cache->row_stride))
    return fail(LCA_ERR_INVALID_ARG, "cache row_stride must be >= 576 and a multiple of 8");
  if (cache->page_rows < 16 || cache->page_rows % 16 != 0)
    return fail(LCA_ERR_UNSUPPORTED, "page_rows = %d: must be a positive multiple of 16", cache->page_rows);
  if (cache->block_table == nullptr || cache->table_stride < 1)
    return fail(LCA_ERR_INVALID_ARG, "block_table must be non-null with table_stride >= 1");
  if (seq_m == nullptr || seq_raw_begin == nullptr || seq_raw_end == nullptr)
    return fail(LCA_ERR_INVALID_ARG, "seq_m, seq_raw_begin and seq_raw_end must be non-null device arrays");
  if (max_entries < 1 || max_entries > ((int64_t)1 << 31)) return fail(LCA_ERR_INVALID_ARG, "max_entries must be in [1, 2^31]");
  if ((rc = check_latent(reps, "reps", true, true)) != LCA_OK) return rc;
  if (reps->dtype != LCA_BF16 || static_cast<const char*>(reps->kr) != static_cast<const char*>(reps->c) + 2 * LCA_D_C ||
      reps->kr_tok_stride != reps->c_tok_stride || reps->kr_seq_stride != reps->c_seq_stride)
    return fail(LCA_ERR_UNSUPPORTED, "paged decode needs packed bf16 representatives (k_R right after c_KV)");
  if (reps->c_tok_stride != cache->row_stride)
    return fail(LCA_ERR_UNSUPPORTED, "representatives and cache pages must share one row stride");
  if (cache->row_stride * 2 * 16 >= ((int64_t)1 << 31)) return fail(LCA_ERR_UNSUPPORTED, "row stride too large");
  if ((rc = check_scale(sm_scale)) != LCA_OK) return rc;
  if (o_latent == nullptr || !aligned16(o_latent)) return fail(LCA_ERR_INVALID_ARG, "o_latent must be a non-null 16-byte aligned pointer");
  const lca::DecodeSplit sp = lca::decode_split(B, lca::head_blocks(H), max_entries);
  *need = lca::decode_workspace_bytes(B, lca::head_blocks(H), sp.S);
  return LCA_OK;
}
}  // namespace

extern "C" {

int mla_latent_attn_decode_paged(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                                 int32_t H, const lca_latent_t* reps, const int32_t* seq_m,
                                 const lca_paged_t* cache, const int32_t* seq_raw_begin,
                                 const int32_t* seq_raw_end, int64_t max_entries, float sm_scale,
                                 float* o_latent, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  const int rc = check_decode_paged(q, q_dtype, q_seq_stride, B, H, reps, seq_m, cache, seq_raw_begin, seq_raw_end,
                                    max_entries, sm_scale, o_latent, &need);
  if (rc != LCA_OK) return rc;
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  return hip_status(lca::launch_decode_paged(q, q_dtype, q_seq_stride, B, H, *reps, seq_m, *cache, seq_raw_begin,
                                             seq_raw_end, max_entries, sm_scale, o_latent, lse, workspace, stream),
                    "mla_latent_attn_decode_paged launch");
}

int mla_latent_attn_decode_paged_up(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                                    int32_t H, const lca_latent_t* reps, const int32_t* seq_m,
                                    const lca_paged_t* cache, const int32_t* seq_raw_begin,
                                    const int32_t* seq_raw_end, int64_t max_entries, float sm_scale,
                                    float* o_latent, float* lse, const void* w_uv, int32_t w_dtype, void* out,
                                    int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  size_t need = 0;
  const int rc = check_decode_paged(q, q_dtype, q_seq_stride, B, H, reps, seq_m, cache, seq_raw_begin, seq_raw_end,
                                    max_entries, sm_scale, o_latent, &need);
  if (rc != LCA_OK) return rc;
  if (!valid_dtype(w_dtype) || !valid_dtype(out_dtype)) return fail(LCA_ERR_INVALID_ARG, "w_dtype and out_dtype must be LCA_BF16 or LCA_F32");
  if (w_uv == nullptr || !aligned16(w_uv) || out == nullptr || !aligned16(out))
    return fail(LCA_ERR_INVALID_ARG, "w_uv and out must be non-null 16-byte aligned pointers");
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  return hip_status(lca::launch_decode_paged_up(q, q_dtype, q_seq_stride, B, H, *reps, seq_m, *cache, seq_raw_begin,
                                                seq_raw_end, max_entries, sm_scale, o_latent, lse, w_uv, w_dtype,
                                                out, out_dtype, workspace, stream),
                    "mla_latent_attn_decode_paged_up launch");
}

int mla_latent_attn_decode_paged_up_step(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                                         int32_t H, const lca_latent_t* reps, int32_t* seq_m,
                                         const lca_paged_t* cache, int32_t* seq_raw_begin, int32_t* seq_raw_end,
                                         int64_t max_entries, float sm_scale, float* o_latent, float* lse,
                                         const void* w_uv, int32_t w_dtype, void* out, int32_t out_dtype,
                                         const lca_step_t* step, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  size_t need = 0;
  int rc = check_decode_paged(q, q_dtype, q_seq_stride, B, H, reps, seq_m, cache, seq_raw_begin, seq_raw_end,
                              max_entries, sm_scale, o_latent, &need);
  if (rc != LCA_OK) return rc;
  if (!valid_dtype(w_dtype) || !valid_dtype(out_dtype)) return fail(LCA_ERR_INVALID_ARG, "w_dtype and out_dtype must be LCA_BF16 or LCA_F32");
  if (w_uv == nullptr || !aligned16(w_uv) || out == nullptr || !aligned16(out))
    return fail(LCA_ERR_INVALID_ARG, "w_uv and out must be non-null 16-byte aligned pointers");
  if (step == nullptr) return fail(LCA_ERR_INVALID_ARG, "step is null");
  if ((rc = check_step(cache, B, step->w, step->g, H, step->q_ring, step->q_ring_seq_stride, reps, step->anchor_idx,
                       step->anchor_seq_stride, seq_m, seq_raw_begin, seq_raw_end)) != LCA_OK)
    return rc;
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  return hip_status(lca::launch_decode_paged_up_step(q, q_dtype, q_seq_stride, B, H, *reps, seq_m, *cache,
                                                     seq_raw_begin, seq_raw_end, max_entries, sm_scale, o_latent, lse,
                                                     w_uv, w_dtype, out, out_dtype, workspace, step->w, step->g,
                                                     step->q_ring, step->q_ring_seq_stride, step->anchor_idx,
                                                     step->anchor_seq_stride, step->pos, step->dst_row, stream),
                    "mla_latent_attn_decode_paged_up_step launch");
}

}  // extern "C"

namespace {
// Arguments of mla_latent_attn_decode_up / _noalloc other than the scratch;
// on success *need receives the bytes of split-K partials the call uses.
int check_decode_up(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B, int32_t H,
                    const lca_latent_t* reps, int64_t m, const lca_latent_t* raw, int64_t raw_begin,
                    int64_t raw_end, float sm_scale, float* o_latent, const void* w_uv, int32_t w_dtype,
                    void* out, int32_t out_dtype, size_t* need) {
  int rc;
  if (q == nullptr || !aligned16(q)) return fail(LCA_ERR_INVALID_ARG, "q must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (!mult8(q_seq_stride) || q_seq_stride < 0) return fail(LCA_ERR_INVALID_ARG, "q_seq_stride must be a non-negative multiple of 8");
  if (B < 1 || B > 65535) return fail(LCA_ERR_INVALID_ARG, "B must be in [1, 65535]");
  if (!lca::heads_supported(H) || lca::head_blocks(H) > 65535)
    return fail(LCA_ERR_UNSUPPORTED, "H = %d: the head count must be a multiple of 16 or divide 16", H);
  if (m < 0 || raw_begin < 0 || raw_end < raw_begin) return fail(LCA_ERR_INVALID_ARG, "need m >= 0 and 0 <= raw_begin <= raw_end");
  const int64_t n = m + (raw_end - raw_begin);
  if (n < 1) return fail(LCA_ERR_INVALID_ARG, "nothing to attend: m + raw_end - raw_begin must be >= 1");
  if (m > 0 && (rc = check_latent(reps, "reps", true, true)) != LCA_OK) return rc;
  if (raw_end > raw_begin && (rc = check_latent(raw, "raw", true, true)) != LCA_OK) return rc;
  if (m > 0 && raw_end > raw_begin && reps->dtype != raw->dtype)
    return fail(LCA_ERR_UNSUPPORTED, "reps and raw must share one dtype");
  if ((rc = check_scale(sm_scale)) != LCA_OK) return rc;
  if (o_latent == nullptr || !aligned16(o_latent)) return fail(LCA_ERR_INVALID_ARG, "o_latent must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(w_dtype) || !valid_dtype(out_dtype)) return fail(LCA_ERR_INVALID_ARG, "w_dtype and out_dtype must be LCA_BF16 or LCA_F32");
  if (w_uv == nullptr || !aligned16(w_uv) || out == nullptr || !aligned16(out))
    return fail(LCA_ERR_INVALID_ARG, "w_uv and out must be non-null 16-byte aligned pointers");
  const lca::DecodeSplit sp = lca::decode_split(B, lca::head_blocks(H), n);
  *need = lca::decode_workspace_bytes(B, lca::head_blocks(H), sp.S);
  return LCA_OK;
}
}  // namespace

extern "C" {

int mla_latent_attn_decode_up(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                              int32_t H, const lca_latent_t* reps, int64_t m,
                              const lca_latent_t* raw, int64_t raw_begin, int64_t raw_end,
                              float sm_scale, float* o_latent, float* lse, const void* w_uv,
                              int32_t w_dtype, void* out, int32_t out_dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  const int rc = check_decode_up(q, q_dtype, q_seq_stride, B, H, reps, m, raw, raw_begin, raw_end, sm_scale,
                                 o_latent, w_uv, w_dtype, out, out_dtype, &need);
  if (rc != LCA_OK) return rc;
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  const lca_latent_t none = {nullptr, nullptr, 0, 0, 0, 0, m > 0 ? reps->dtype : raw->dtype};
  const lca_latent_t& rp = m > 0 ? *reps : none;
  const lca_latent_t& rw = raw_end > raw_begin ? *raw : none;
  return hip_status(lca::launch_decode_up(q, q_dtype, q_seq_stride, B, H, rp, m, rw, raw_begin, raw_end,
                                          sm_scale, o_latent, lse, w_uv, w_dtype, out, out_dtype,
                                          workspace, stream),
                    "mla_latent_attn_decode_up launch");
}

int mla_latent_attn_decode_up_noalloc(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                                      int32_t H, const lca_latent_t* reps, int64_t m,
                                      const lca_latent_t* raw, int64_t raw_begin, int64_t raw_end,
                                      float sm_scale, float* o_latent, float* lse, const void* w_uv,
                                      int32_t w_dtype, void* out, int32_t out_dtype, hipStream_t stream) {
  size_t need = 0;
  const int rc = check_decode_up(q, q_dtype, q_seq_stride, B, H, reps, m, raw, raw_begin, raw_end, sm_scale,
                                 o_latent, w_uv, w_dtype, out, out_dtype, &need);
  if (rc != LCA_OK) return rc;
  if (need > LCA_NOALLOC_SCRATCH_BYTES)
    return fail(LCA_ERR_UNSUPPORTED, "this call needs %zu bytes of split-K scratch; the library's fixed scratch "
                "holds %zu", need, (size_t)LCA_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  if (need > 0) {
    const int st = hip_status(lca::noalloc_scratch(&scratch), "scratch address lookup");
    if (st != LCA_OK) return st;
  }
  const lca_latent_t none = {nullptr, nullptr, 0, 0, 0, 0, m > 0 ? reps->dtype : raw->dtype};
  const lca_latent_t& rp = m > 0 ? *reps : none;
  const lca_latent_t& rw = raw_end > raw_begin ? *raw : none;
  return hip_status(lca::launch_decode_up(q, q_dtype, q_seq_stride, B, H, rp, m, rw, raw_begin, raw_end,
                                          sm_scale, o_latent, lse, w_uv, w_dtype, out, out_dtype,
                                          scratch, stream),
                    "mla_latent_attn_decode_up_noalloc launch");
}

static int prefill_dense(const void* q, int32_t q_dtype, int64_t q_tok_stride, int64_t chunk_start, int32_t C,
                         int32_t H, const lca_latent_t* reps, int64_t m, const lca_latent_t* raw,
                         int64_t raw_begin, float sm_scale, void* o_latent, int32_t o_dtype, float* lse,
                         int32_t* sched, hipStream_t stream) {
  int rc;
  if (q == nullptr || !aligned16(q)) return fail(LCA_ERR_INVALID_ARG, "q must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (!mult8(q_tok_stride) || q_tok_stride < 0) return fail(LCA_ERR_INVALID_ARG, "q_tok_stride must be a non-negative multiple of 8");
  if (C < 1) return fail(LCA_ERR_INVALID_ARG, "C must be >= 1");
  if (!lca::heads_supported(H) || lca::head_blocks(H) > 65535)
    return fail(LCA_ERR_UNSUPPORTED, "H = %d: the head count must be a multiple of 16 or divide 16", H);
  if (m < 0 || raw_begin < 0 || chunk_start < raw_begin)
    return fail(LCA_ERR_INVALID_ARG, "need m >= 0 and 0 <= raw_begin <= chunk_start");
  if (m > 0 && (rc = check_latent(reps, "reps", true, true)) != LCA_OK) return rc;
  if ((rc = check_latent(raw, "raw", true, true)) != LCA_OK) return rc;
  if (m > 0 && reps->dtype != raw->dtype) return fail(LCA_ERR_UNSUPPORTED, "reps and raw must share one dtype");
  if ((rc = check_scale(sm_scale)) != LCA_OK) return rc;
  if (!valid_dtype(o_dtype)) return fail(LCA_ERR_INVALID_ARG, "o_dtype %d is not LCA_BF16/LCA_F32", o_dtype);
  if (o_latent == nullptr || !aligned16(o_latent)) return fail(LCA_ERR_INVALID_ARG, "o_latent must be a non-null 16-byte aligned pointer");
  const lca_latent_t none = {nullptr, nullptr, 0, 0, 0, 0, raw->dtype};
  return hip_status(lca::launch_prefill(q, q_dtype, q_tok_stride, chunk_start, C, H, m > 0 ? *reps : none,
                                        m, *raw, raw_begin, sm_scale, o_latent, o_dtype, lse, stream, sched),
                    "mla_latent_attn_prefill_chunk launch");
}

int mla_latent_attn_prefill_chunk(const void* q, int32_t q_dtype, int64_t q_tok_stride,
                                  int64_t chunk_start, int32_t C, int32_t H,
                                  const lca_latent_t* reps, int64_t m,
                                  const lca_latent_t* raw, int64_t raw_begin, float sm_scale,
                                  void* o_latent, int32_t o_dtype, float* lse,
                                  hipStream_t stream) {
  return prefill_dense(q, q_dtype, q_tok_stride, chunk_start, C, H, reps, m, raw, raw_begin, sm_scale, o_latent,
                       o_dtype, lse, nullptr, stream);
}

int mla_latent_attn_prefill_chunk_sched(const void* q, int32_t q_dtype, int64_t q_tok_stride,
                                        int64_t chunk_start, int32_t C, int32_t H,
                                        const lca_latent_t* reps, int64_t m,
                                        const lca_latent_t* raw, int64_t raw_begin, float sm_scale,
                                        void* o_latent, int32_t o_dtype, float* lse,
                                        int32_t* sched, hipStream_t stream) {
  if (sched == nullptr || reinterpret_cast<uintptr_t>(sched) % 8 != 0)
    return fail(LCA_ERR_INVALID_ARG, "sched must be a non-null 8-byte aligned pointer to two int32");
  return prefill_dense(q, q_dtype, q_tok_stride, chunk_start, C, H, reps, m, raw, raw_begin, sm_scale, o_latent,
                       o_dtype, lse, sched, stream);
}

static int prefill_paged(const void* q, int32_t q_dtype, int64_t q_tok_stride, int64_t chunk_start, int32_t C,
                         int32_t H, const lca_latent_t* reps, int64_t m, const lca_paged_t* cache, int32_t seq,
                         int64_t raw_begin, float sm_scale, void* o_latent, int32_t o_dtype, float* lse,
                         int32_t* sched, hipStream_t stream) {
  int rc;
  if (q == nullptr || !aligned16(q)) return fail(LCA_ERR_INVALID_ARG, "q must be a non-null 16-byte aligned pointer");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (!mult8(q_tok_stride) || q_tok_stride < 0) return fail(LCA_ERR_INVALID_ARG, "q_tok_stride must be a non-negative multiple of 8");
  if (C < 1) return fail(LCA_ERR_INVALID_ARG, "C must be >= 1");
  if (!lca::heads_supported(H) || lca::head_blocks(H) > 65535)
    return fail(LCA_ERR_UNSUPPORTED, "H = %d: the head count must be a multiple of 16 or divide 16", H);
  if (m < 0 || raw_begin < 0 || chunk_start < raw_begin)
    return fail(LCA_ERR_INVALID_ARG, "need m >= 0 and 0 <= raw_begin <= chunk_start");
  if (cache == nullptr || cache->pages == nullptr || !aligned16(cache->pages))
    return fail(LCA_ERR_INVALID_ARG, "cache pages must be a non-null 16-byte aligned pointer");
  if (cache->row_stride < LCA_D_ROW || !mult8(cache->row_stride))
    return fail(LCA_ERR_INVALID_ARG, "cache row_stride must be >= 576 and a multiple of 8");
  if (cache->page_rows < 16 || cache->page_rows % 16 != 0)
    return fail(LCA_ERR_UNSUPPORTED, "page_rows = %d: must be a positive multiple of 16", cache->page_rows);
  if (cache->block_table == nullptr || cache->table_stride < 1)
    return fail(LCA_ERR_INVALID_ARG, "block_table must be non-null with table_stride >= 1");
  if (seq < 0) return fail(LCA_ERR_INVALID_ARG, "seq must be >= 0");
  if (cache->row_stride * 2 * 32 >= ((int64_t)1 << 31)) return fail(LCA_ERR_UNSUPPORTED, "row stride too large");
  if (m > 0) {
    if ((rc = check_latent(reps, "reps", true, true)) != LCA_OK) return rc;
    if (reps->dtype != LCA_BF16 || static_cast<const char*>(reps->kr) != static_cast<const char*>(reps->c) + 2 * LCA_D_C ||
        reps->kr_tok_stride != reps->c_tok_stride)
      return fail(LCA_ERR_UNSUPPORTED, "paged prefill needs packed bf16 representatives (k_R right after c_KV)");
    if (reps->c_tok_stride != cache->row_stride)
      return fail(LCA_ERR_UNSUPPORTED, "representatives and cache pages must share one row stride");
  }
  if ((rc = check_scale(sm_scale)) != LCA_OK) return rc;
  if (!valid_dtype(o_dtype)) return fail(LCA_ERR_INVALID_ARG, "o_dtype %d is not LCA_BF16/LCA_F32", o_dtype);
  if (o_latent == nullptr || !aligned16(o_latent)) return fail(LCA_ERR_INVALID_ARG, "o_latent must be a non-null 16-byte aligned pointer");
  const lca_latent_t none = {nullptr, nullptr, 0, 0, 0, 0, LCA_BF16};
  return hip_status(lca::launch_prefill_paged(q, q_dtype, q_tok_stride, chunk_start, C, H, m > 0 ? *reps : none, m,
                                              *cache, seq, raw_begin, sm_scale, o_latent, o_dtype, lse, stream,
                                              sched),
                    "mla_latent_attn_prefill_chunk_paged launch");
}

int mla_latent_attn_prefill_chunk_paged(const void* q, int32_t q_dtype, int64_t q_tok_stride,
                                        int64_t chunk_start, int32_t C, int32_t H,
                                        const lca_latent_t* reps, int64_t m, const lca_paged_t* cache,
                                        int32_t seq, int64_t raw_begin, float sm_scale, void* o_latent,
                                        int32_t o_dtype, float* lse, hipStream_t stream) {
  return prefill_paged(q, q_dtype, q_tok_stride, chunk_start, C, H, reps, m, cache, seq, raw_begin, sm_scale,
                       o_latent, o_dtype, lse, nullptr, stream);
}

int mla_latent_attn_prefill_chunk_paged_sched(const void* q, int32_t q_dtype, int64_t q_tok_stride,
                                              int64_t chunk_start, int32_t C, int32_t H,
                                              const lca_latent_t* reps, int64_t m, const lca_paged_t* cache,
                                              int32_t seq, int64_t raw_begin, float sm_scale, void* o_latent,
                                              int32_t o_dtype, float* lse, int32_t* sched, hipStream_t stream) {
  if (sched == nullptr || reinterpret_cast<uintptr_t>(sched) % 8 != 0)
    return fail(LCA_ERR_INVALID_ARG, "sched must be a non-null 8-byte aligned pointer to two int32");
  return prefill_paged(q, q_dtype, q_tok_stride, chunk_start, C, H, reps, m, cache, seq, raw_begin, sm_scale,
                       o_latent, o_dtype, lse, sched, stream);
}

int mla_up_proj(const void* o_latent, int32_t o_dtype, int64_t T, int32_t H, const void* w_uv,
                int32_t w_dtype, void* out, int32_t out_dtype, hipStream_t stream) {
  if (T < 0) return fail(LCA_ERR_INVALID_ARG, "T must be >= 0");
  if (H < 1 || H > 65535) return fail(LCA_ERR_INVALID_ARG, "H must be in [1, 65535]");
  if (!valid_dtype(o_dtype) || !valid_dtype(w_dtype) || !valid_dtype(out_dtype))
    return fail(LCA_ERR_INVALID_ARG, "dtypes must be LCA_BF16 or LCA_F32");
  if (T == 0) return ok();
  if (o_latent == nullptr || !aligned16(o_latent) || w_uv == nullptr || !aligned16(w_uv) ||
      out == nullptr || !aligned16(out))
    return fail(LCA_ERR_INVALID_ARG, "o_latent, w_uv and out must be non-null 16-byte aligned pointers");
  if ((T + 63) / 64 > 0x7fffffff) return fail(LCA_ERR_UNSUPPORTED, "T too large");
  return hip_status(lca::launch_up_proj(o_latent, o_dtype, T, H, w_uv, w_dtype, out, out_dtype, stream),
                    "mla_up_proj launch");
}

size_t lca_project_workspace_size(int64_t T, int32_t H) {
  if (T < 0 || H < 1) return 0;
  return (size_t)T * (size_t)H * LCA_D_V * 2;  // q^nope of every token and head, bf16
}

int lca_project(const void* x, int64_t x_tok_stride, int64_t T, int32_t d_model, const int32_t* pos,
                double rope_base, const void* w_proj, const void* w_uk, int32_t H, void* rows,
                int64_t row_stride, const int64_t* dst_row, void* q, int32_t q_dtype, int64_t q_tok_stride,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0) return fail(LCA_ERR_INVALID_ARG, "T must be >= 0");
  if (H < 1 || H > 1024) return fail(LCA_ERR_UNSUPPORTED, "H = %d: supported head counts are 1..1024", H);
  if (d_model < 32 || d_model % 32 != 0)
    return fail(LCA_ERR_UNSUPPORTED, "d_model = %d: must be a positive multiple of 32", d_model);
  if (!(std::isfinite(rope_base) && rope_base > 1.0)) return fail(LCA_ERR_INVALID_ARG, "rope_base must be finite and > 1");
  if (!valid_dtype(q_dtype)) return fail(LCA_ERR_INVALID_ARG, "q_dtype %d is not LCA_BF16/LCA_F32", q_dtype);
  if (T == 0) return ok();
  if (x == nullptr || !aligned16(x) || w_proj == nullptr || !aligned16(w_proj) || w_uk == nullptr ||
      !aligned16(w_uk))
    return fail(LCA_ERR_INVALID_ARG, "x, w_proj and w_uk must be non-null 16-byte aligned pointers");
  if (x_tok_stride < d_model || !mult8(x_tok_stride))
    return fail(LCA_ERR_INVALID_ARG, "x_tok_stride must be >= d_model and a multiple of 8");
  if (pos == nullptr || dst_row == nullptr) return fail(LCA_ERR_INVALID_ARG, "pos and dst_row must be non-null device arrays");
  if (rows == nullptr || !aligned16(rows) || row_stride < LCA_D_ROW || !mult8(row_stride))
    return fail(LCA_ERR_INVALID_ARG, "rows must be non-null and aligned, row_stride >= 576 and a multiple of 8");
  if (q == nullptr || !aligned16(q) || q_tok_stride < (int64_t)H * LCA_D_ROW || !mult8(q_tok_stride))
    return fail(LCA_ERR_INVALID_ARG, "q must be non-null and aligned, q_tok_stride >= 576 H and a multiple of 8");
  const size_t need = lca_project_workspace_size(T, H);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return fail(LCA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  if ((T + 127) / 128 > 0x7fffffff) return fail(LCA_ERR_UNSUPPORTED, "T too large");
  return hip_status(lca::launch_project(x, x_tok_stride, T, d_model, pos, rope_base, w_proj, w_uk, H, rows,
                                        row_stride, dst_row, q, q_dtype, q_tok_stride, workspace, stream),
                    "lca_project launch");
}

}  // extern "C"
