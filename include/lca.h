/* lca.h - C ABI of the latent-condensed MLA kernels for MI355X (gfx950).
 *
 * The method is Latent-Condensed Attention (LCA) as described on the page
 * "Latent-Condensed Transformer for Efficient Long Context Modeling"
 * (papernotes.org notes on the ACL 2026 paper, arXiv 2604.12452), run directly
 * over a Multi-head Latent Attention (MLA) cache as described on the page
 * "新一代开源大模型架构演进与注意力机制深度对比解析" (cloud.baidu.com), section
 * 三.1: every token caches a latent row and heads project it back up at
 * compute time.
 *
 * A cached token is one row of a 512-wide latent c_KV and a 64-wide decoupled
 * RoPE key k_R (the page's C^KV and K^R, 研究背景 / 核心矛盾). The history older
 * than the last w tokens is cut into m = floor((L - w) / g) groups of g tokens
 * (方法详解 / 整体框架). Each group becomes one representative row: its c_KV is
 * the softmax-weighted sum of the group's c_KV rows, weighted by the
 * importance of each token to the summary query (关键设计 1), and its k_R is
 * the k_R of the group's most important token (关键设计 2). Attention then runs
 * over [representatives ++ the uncompressed rows] (整体框架, flowchart E -> F).
 *
 * Conventions shared by every call:
 *  - Device buffers are owned by the caller. The library never allocates or
 *    frees device memory; scratch space comes from a caller workspace (the
 *    one exception, mla_latent_attn_decode_up_noalloc, uses a fixed device
 *    array that the library holds per GPU).
 *  - Inputs are never written. Outputs are fully written, except that
 *    lca_condense writes only the representative rows it is asked for.
 *  - Calls are asynchronous on `stream` (a hipStream_t; 0 = the null stream)
 *    and never synchronise. Argument errors are returned synchronously as a
 *    negative lca_status_t with text from lca_last_error(); a launch failure
 *    returns LCA_ERR_HIP. Device faults surface at the caller's next sync.
 *  - Strides are in elements. Row starts must be 16-byte aligned and token
 *    strides multiples of 8 elements (vectorised 16-byte loads).
 *  - bf16 values are stored as raw bfloat16; f32 inputs of the attention
 *    paths are rounded to bf16 (nearest even) where they feed the matrix
 *    cores. Accumulation is fp32 everywhere.
 *  - Results are bitwise deterministic for fixed inputs and arguments.
 */
#ifndef LCA_H_
#define LCA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCA_VERSION 1004 /* major*1000 + minor */
#define LCA_D_C 512      /* latent c_KV width */
#define LCA_D_R 64       /* decoupled RoPE key width */
#define LCA_D_ROW 576    /* one cached row: c_KV ++ k_R */
#define LCA_D_V 128      /* per-head value width of W_UV */
#define LCA_MAX_G 32     /* largest supported group size (powers of two): one
                          * wavefront holds a whole group in registers, 8
                          * latent columns of every row per lane; the pages
                          * use g = 16 throughout (局限与展望 names the fixed
                          * g as a limitation) */

typedef enum {
  LCA_OK = 0,
  LCA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, out-of-range rows */
  LCA_ERR_UNSUPPORTED = -2, /* a size the kernels are not built for (e.g. H = 24) */
  LCA_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required */
  LCA_ERR_HIP = -4          /* the HIP runtime refused a launch */
} lca_status_t;

typedef enum { LCA_BF16 = 0, LCA_F32 = 1 } lca_dtype_t;

/* A latent cache (or representative) tensor of B sequences.
 * c_KV of token t of sequence b starts at  c  + b*c_seq_stride  + t*c_tok_stride,
 * k_R  of token t of sequence b starts at  kr + b*kr_seq_stride + t*kr_tok_stride.
 * A packed [B, L, 576] buffer is c = base, kr = base + 512 with equal strides. */
typedef struct {
  void* c;
  void* kr;
  int64_t c_seq_stride, c_tok_stride;
  int64_t kr_seq_stride, kr_tok_stride;
  int32_t dtype; /* lca_dtype_t, shared by c and kr */
} lca_latent_t;

/* Grouping of a cache of L tokens: m groups [j g, (j+1) g) for j < m, raw rows
 * [raw_begin, raw_end) = [m g, L), n_entries = m + (L - m g) attended rows. */
typedef struct {
  int64_t m, raw_begin, raw_end, n_entries;
} lca_plan_t;

int lca_version(void);

/* Text of the last error on the calling thread ("" after success). */
const char* lca_last_error(void);

/* Host-only. m = floor((L - w) / g) when L > w, else 0 (方法详解 / 整体框架);
 * the (L - w) mod g tokens left over stay raw. L, w >= 0, 1 <= g. */
int lca_plan(int64_t L, int64_t w, int32_t g, lca_plan_t* out);

/* Workspace bytes lca_condense needs: one fp32 summary query per sequence
 * and group (q_row_step > 0), or per sequence plus 8 fp32 partial sums of
 * its query rows (q_row_step == 0). */
size_t lca_condense_workspace_size(int32_t B, int64_t n_groups, int64_t q_row_step);

/* Condense groups [group_begin, group_begin + n_groups) of every sequence
 * (关键设计 1 and 关键设计 2).
 *
 *  cache        c_KV / k_R of the token rows; group j reads tokens [j g, (j+1) g).
 *  g            group size: a power of two, 1 <= g <= LCA_MAX_G.
 *  q            absorbed queries [B, T, H, 576] (row t, head h of sequence b at
 *               q + b*q_seq_stride + t*q_tok_stride + h*576), dtype q_dtype.
 *  q_row0,      group group_begin + n takes its summary query from query rows
 *  q_row_step   [q_row0 + n*q_row_step, ... + g): the mean over those g tokens
 *               and all H heads (the page's mean of the most recent g queries).
 *               Decode uses q_row_step = 0 (one shared summary query); chunked
 *               prefill uses q_row0 = (group_begin + 1) g, q_row_step = g (the g
 *               queries that follow each group). All rows must lie in [0, T).
 *  sm_scale     >= 0. Importance s_i = qbar . [c_i ; k_R_i]; weights
 *               alpha = softmax(sm_scale * s) over the group.
 *  reps         receives row j (for j in the range) of every sequence:
 *               c_rep = sum_i alpha_i c_i (fp32 accumulation, stored in
 *               reps->dtype) and k_rep = k_R of the anchor I_j.
 *  anchor_idx   int32 [B, *]: anchor_idx[b*anchor_seq_stride + j] = I_j, the
 *               absolute token index of the group's largest score (lowest
 *               index on ties).
 *  alpha        optional fp32 [B, *, g]: alpha[b*alpha_seq_stride + j*g + i].
 *  workspace    >= lca_condense_workspace_size(B, n_groups, q_row_step) bytes,
 *               16-byte aligned; overwritten.
 * n_groups == 0 is a no-op. */
int lca_condense(const lca_latent_t* cache, int32_t B, int32_t g, int64_t group_begin,
                 int64_t n_groups, const void* q, int32_t q_dtype, int64_t q_seq_stride,
                 int64_t q_tok_stride, int64_t T, int32_t H, int64_t q_row0,
                 int64_t q_row_step, float sm_scale, const lca_latent_t* reps,
                 int32_t* anchor_idx, int64_t anchor_seq_stride, float* alpha,
                 int64_t alpha_seq_stride, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Condensation modes. LCA_MODE_LCA is the method (关键设计 1 and 2: latent
 * rows pooled with the softmax weights, RoPE key of the most important
 * token). The other two are the variants of the ablation table (消融实验):
 * LCA_MODE_POOL_ROPE pools the RoPE keys with the same weights as the
 * latents ("pure pooling including position"); LCA_MODE_ANCHOR keeps the
 * most important token's whole row ("pure sparse"). */
typedef enum { LCA_MODE_LCA = 0, LCA_MODE_POOL_ROPE = 1, LCA_MODE_ANCHOR = 2 } lca_mode_t;

/* lca_condense with an explicit mode (lca_condense is mode LCA_MODE_LCA).
 * Same arguments, layouts, ownership and errors; a mode outside lca_mode_t
 * returns LCA_ERR_INVALID_ARG. alpha and the anchor index are the same in
 * every mode; in LCA_MODE_ANCHOR the representative is a bit-exact copy of
 * the anchor row (converted to the representatives' dtype). */
int lca_condense_mode(const lca_latent_t* cache, int32_t B, int32_t g, int64_t group_begin,
                      int64_t n_groups, const void* q, int32_t q_dtype, int64_t q_seq_stride,
                      int64_t q_tok_stride, int64_t T, int32_t H, int64_t q_row0,
                      int64_t q_row_step, float sm_scale, const lca_latent_t* reps,
                      int32_t* anchor_idx, int64_t anchor_seq_stride, float* alpha,
                      int64_t alpha_seq_stride, void* workspace, size_t workspace_bytes,
                      int32_t mode, hipStream_t stream);

/* A paged latent cache for ragged batches: packed bf16 rows [c_KV (512) ++
 * k_R (64)] stored in fixed-size pages of a shared pool. Token t of sequence
 * b is row t % page_rows of page block_table[b * table_stride + t / page_rows],
 * at pages + (page * page_rows + t % page_rows) * row_stride (elements).
 * page_rows is a multiple of 16; block_table is a device int32 array. */
typedef struct {
  const void* pages;
  int64_t row_stride;            /* elements between rows, >= 576, multiple of 8 */
  int32_t page_rows;
  const int32_t* block_table;
  int64_t table_stride;          /* block_table entries per sequence */
} lca_paged_t;

/* lca_condense over a ragged batch with a paged cache (lca_paged_t
 * above): for every sequence b, groups j = seq_group_begin[b] + n, n in
 * [0, seq_n_groups[b]) (tokens [j g, (j+1) g) read through the block table)
 * are condensed as in lca_condense, group j with the summary query of query
 * rows [q_row0 + n q_row_step, + g) of sequence b (the mean over those g
 * tokens and the H heads). q_row_step = 0 gives every group of a sequence
 * the same summary query (decode: the most recent g queries); q_row_step = g
 * with q_row0 = (seq_group_begin + 1) g gives each group the g queries that
 * follow it (chunked prefill, 整体框架 as for mla_latent_attn_prefill_chunk).
 * The rows must lie in [0, T) for every n < max_groups. Representative j is written to row j of reps
 * (packed bf16, dense, row b at reps->c + b * reps->c_seq_stride); anchors
 * are absolute token indices; alpha optional as in lca_condense.
 * seq_group_begin and seq_n_groups are device int32 [B] arrays read only by
 * the kernel; the caller guarantees 0 <= seq_n_groups[b] <= max_groups, that
 * the representative rows exist and that the block table maps every token
 * of the groups. page_rows must be a multiple of g (a group never straddles
 * pages). workspace >= lca_condense_workspace_size(B, max_groups,
 * q_row_step). */
int lca_condense_paged(const lca_paged_t* cache, int32_t B, int32_t g, const int32_t* seq_group_begin,
                       const int32_t* seq_n_groups, int64_t max_groups, const void* q, int32_t q_dtype,
                       int64_t q_seq_stride, int64_t q_tok_stride, int64_t T, int32_t H, int64_t q_row0,
                       int64_t q_row_step, float sm_scale, const lca_latent_t* reps, int32_t* anchor_idx,
                       int64_t anchor_seq_stride, float* alpha, int64_t alpha_seq_stride,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One decode step's incremental condensation over a ragged batch on a
 * paged cache, with the per-sequence state kept on the device, so that a
 * decode step (lca_project, mla_latent_attn_decode_paged[_up], then this
 * call) is the same launch sequence every step and a graph of one step can
 * be replayed. 关键设计 1: a group is condensed with the mean of the most
 * recent g queries once it leaves the window (reading R7: representatives
 * are frozen afterwards).
 *
 * State of sequence b, device int32 [B] arrays (read and rewritten):
 *   seq_raw_end[b]   L: cache tokens before this step's row. The step's row
 *                    (token L) has been written to the cache by the caller,
 *                    after the step's attention read [seq_raw_begin, L).
 *   seq_m[b]         m: representatives so far; seq_raw_begin[b] = m g.
 * For every b this call (one launch):
 *   1. writes this step's query q[b] ([H, 576], q + b*q_seq_stride) to row
 *      L mod g of the sequence's query ring (q_ring + b*q_ring_seq_stride,
 *      g rows of [H, 576], contiguous, same dtype as q). Ring row j holds
 *      the query of the latest token t = j (mod g); the caller fills it for
 *      the g tokens before the first step;
 *   2. if L + 1 - w >= (m + 1) g, condenses group m (tokens [m g, (m+1) g),
 *      through the block table) with the mean over the g ring rows and the
 *      H heads as its summary query, exactly as lca_condense_paged: the
 *      representative goes to row m of reps (packed bf16 rows, sequence b
 *      at reps->c + b * reps->c_seq_stride), the anchor (absolute token
 *      index) to anchor_idx[b * anchor_seq_stride + m]; then m = m + 1;
 *   3. writes the next step's state: seq_m = m, seq_raw_begin = m g,
 *      seq_raw_end = L + 1, and, when non-null, pos[b] = L + 1 (int32) and
 *      dst_row[b] (int64) = the pool row of token L + 1 through the block
 *      table (-1 when token L + 1 lies past table_stride pages), which is
 *      what lca_project needs for the next token.
 * The caller guarantees that the block table maps every token read, that
 * reps and anchor_idx have a row for every group condensed, and that the
 * state is consistent (seq_raw_begin = seq_m g); out-of-range state is not
 * detected. page_rows must be a multiple of g. Errors as for the other
 * calls; nothing is allocated. */
int lca_condense_step(const lca_paged_t* cache, int32_t B, int64_t w, int32_t g, const void* q,
                      int32_t q_dtype, int64_t q_seq_stride, int32_t H, void* q_ring,
                      int64_t q_ring_seq_stride, float sm_scale, const lca_latent_t* reps,
                      int32_t* anchor_idx, int64_t anchor_seq_stride, int32_t* seq_m,
                      int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos, int64_t* dst_row,
                      hipStream_t stream);

/* Workspace bytes mla_latent_attn_decode needs for up to max_entries
 * attended rows per sequence (split-K partial results). */
size_t mla_latent_attn_decode_workspace_size(int32_t B, int32_t H, int64_t max_entries);

/* One decode step of MLA attention over a condensed latent cache
 * (整体框架, flowchart E -> F: representatives concatenated with the window,
 * then standard attention).
 *
 *  q        absorbed queries [B, H, 576] (head h of sequence b at
 *           q + b*q_seq_stride + h*576). H is a multiple of 16, or 1, 2,
 *           4 or 8 (one head group of grouped-query attention: one latent
 *           cache per key-value head, attended by its Hg query heads, run
 *           as B * n_kv sequences of Hg heads each).
 *  reps     entries [0, m) of each sequence are representative rows 0..m-1.
 *  raw      entries [m, m + raw_end - raw_begin) are cache rows
 *           [raw_begin, raw_end). reps->dtype must equal raw->dtype.
 *           Plain MLA is m = 0, raw = [0, L).
 *  For every head: z_e = sm_scale * q_h . [c_e ; k_R_e], p = softmax(z),
 *  o_latent[b, h, :] = sum_e p_e c_e  (fp32 [B, H, 512], contiguous) and
 *  lse[b, h] = log(sum_e exp(z_e))    (fp32 [B, H], optional).
 *  The per-head value is o_latent[b, h] @ W_UV[h] (mla_up_proj).
 *  workspace >= mla_latent_attn_decode_workspace_size(B, H, m + raw_end -
 *  raw_begin) bytes, 16-byte aligned, owned by the caller. When the entries
 *  are split across several workgroups it holds their partial results
 *  (per split: running max and sum, then the unnormalised 512-wide output),
 *  which a second kernel merges; every value read there was written by the
 *  same call, so no initialisation is needed. Calls that run concurrently
 *  must not share a workspace. */
int mla_latent_attn_decode(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                           int32_t H, const lca_latent_t* reps, int64_t m,
                           const lca_latent_t* raw, int64_t raw_begin, int64_t raw_end,
                           float sm_scale, float* o_latent, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Decode over a ragged batch with a paged cache (a serving layout; the
 * attention is that of mla_latent_attn_decode, 整体框架 flowchart E -> F).
 * Sequence b attends representative rows [0, seq_m[b]) of reps (dense,
 * packed bf16, row b at reps->c + b * reps->c_seq_stride) followed by its
 * cache tokens [seq_raw_begin[b], seq_raw_end[b]) read through the block
 * table. seq_m, seq_raw_begin, seq_raw_end are device int32 [B] arrays,
 * read only by the kernel; the caller guarantees for every b: 0 <=
 * seq_raw_begin <= seq_raw_end, seq_m + (seq_raw_end - seq_raw_begin) in
 * [1, max_entries], the representative rows exist, and the block table maps
 * every token in the raw range to a page of the pool (out-of-range values
 * are not detected and read arbitrary memory). reps->c_tok_stride must equal
 * cache->row_stride. q, o_latent, lse as in mla_latent_attn_decode;
 * workspace >= mla_latent_attn_decode_workspace_size(B, H, max_entries).
 * Outputs are not bitwise equal to the dense entry point's (tiles are
 * formed differently), only within rounding. */
int mla_latent_attn_decode_paged(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                                 int32_t H, const lca_latent_t* reps, const int32_t* seq_m,
                                 const lca_paged_t* cache, const int32_t* seq_raw_begin,
                                 const int32_t* seq_raw_end, int64_t max_entries, float sm_scale,
                                 float* o_latent, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* mla_latent_attn_decode_paged followed by mla_up_proj of its output (a
 * serving layout; the MLA page's projection back to each head's value space,
 * 三.1), with the split merge and the projection fused as in
 * mla_latent_attn_decode_up. Arguments as in mla_latent_attn_decode_paged
 * plus w_uv [H, 512, 128] contiguous (w_dtype) and out [B, H, 128]
 * contiguous (out_dtype). The results are bitwise equal to the two calls in
 * sequence; workspace as for mla_latent_attn_decode_paged. */
int mla_latent_attn_decode_paged_up(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                                    int32_t H, const lca_latent_t* reps, const int32_t* seq_m,
                                    const lca_paged_t* cache, const int32_t* seq_raw_begin,
                                    const int32_t* seq_raw_end, int64_t max_entries, float sm_scale,
                                    float* o_latent, float* lse, const void* w_uv, int32_t w_dtype, void* out,
                                    int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* The step condensation of lca_condense_step as the tail of a paged decode
 * with W_UV (a serving layout: one decode step is then two calls,
 * lca_project and this one, the same every step). Fields as the arguments
 * of lca_condense_step of the same names; pos and dst_row may be null. */
typedef struct {
  int64_t w;                  /* window */
  int32_t g;                  /* group size */
  void* q_ring;               /* [B, g, H, 576] query ring, q's dtype */
  int64_t q_ring_seq_stride;  /* elements between sequences of the ring */
  int32_t* anchor_idx;
  int64_t anchor_seq_stride;
  int32_t* pos;               /* out: next token's position, int32 [B] */
  int64_t* dst_row;           /* out: next token's pool row, int64 [B] */
} lca_step_t;

/* mla_latent_attn_decode_paged_up, then lca_condense_step with this step's
 * queries q and the same reps, cache, seq_m, seq_raw_begin, seq_raw_end and
 * sm_scale (整体框架 for the attention, 关键设计 1 for the condensation).
 * The per-sequence arrays are read by the attention and then rewritten for
 * the next step, so they are not const here. For B <= 64 the condensation
 * runs as extra workgroups of the W_UV up-projection kernel, which follows
 * the attention kernel, so the step costs no launch of its own; for larger
 * batches it is launched after the projection. Results are bitwise those of
 * the two calls in sequence. Workspace as for mla_latent_attn_decode_paged. */
int mla_latent_attn_decode_paged_up_step(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                                         int32_t H, const lca_latent_t* reps, int32_t* seq_m,
                                         const lca_paged_t* cache, int32_t* seq_raw_begin,
                                         int32_t* seq_raw_end, int64_t max_entries, float sm_scale,
                                         float* o_latent, float* lse, const void* w_uv, int32_t w_dtype,
                                         void* out, int32_t out_dtype, const lca_step_t* step,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* mla_latent_attn_decode followed by mla_up_proj of its output (the MLA
 * page's projection back to each head's value space, 三.1), with the split
 * merge and the projection fused into one kernel when B <= 64 and the
 * entries are split 2 to 32 ways (otherwise they run as two kernels, or the
 * projection alone when there is one split). Arguments as
 * in the two calls: o_latent and lse receive the decode results,
 * out[b, h, :] = o_latent[b, h, :] @ W_UV[h] (w_uv [H, 512, 128] contiguous,
 * out [B, H, 128] contiguous, dtypes w_dtype / out_dtype). The results are
 * bitwise equal to the two calls in sequence. workspace as for
 * mla_latent_attn_decode (same size). */
int mla_latent_attn_decode_up(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                              int32_t H, const lca_latent_t* reps, int64_t m,
                              const lca_latent_t* raw, int64_t raw_begin, int64_t raw_end,
                              float sm_scale, float* o_latent, float* lse, const void* w_uv,
                              int32_t w_dtype, void* out, int32_t out_dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Bytes of device scratch the library keeps for
 * mla_latent_attn_decode_up_noalloc on every GPU it runs on (16 MiB; every
 * split plan of the decode calls fits). */
#define LCA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* mla_latent_attn_decode_up for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments, layouts, results (bitwise equal
 * to mla_latent_attn_decode_up on the same inputs) and errors, without the
 * workspace argument. The split-K partial results live instead in a
 * file-scope device array of LCA_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU until the process ends; its address is looked up once per
 * device, on the first call with that device current. The call allocates
 * nothing and never synchronises. A shape whose partial results would exceed
 * the array returns LCA_ERR_UNSUPPORTED (none of the decode split plans
 * does). Every call on one GPU shares that GPU's array and leaves the last
 * call's partials in it; no value is read there before the same call wrote
 * it, so nothing needs clearing. Calls that overlap on one GPU (several
 * streams, or threads without ordering) race on the array and must not be
 * issued. */
int mla_latent_attn_decode_up_noalloc(const void* q, int32_t q_dtype, int64_t q_seq_stride, int32_t B,
                                      int32_t H, const lca_latent_t* reps, int64_t m,
                                      const lca_latent_t* raw, int64_t raw_begin, int64_t raw_end,
                                      float sm_scale, float* o_latent, float* lse, const void* w_uv,
                                      int32_t w_dtype, void* out, int32_t out_dtype, hipStream_t stream);

/* Chunked prefill attention of one sequence over a condensed latent cache
 * ("Latent-Condensed Transformer for Efficient Long Context Modeling",
 * 方法详解 / 整体框架 and its flowchart E -> F: each query attends to the
 * representatives of the groups older than its local window plus the
 * uncompressed rows of the window; the pages give no prefill-specific rule,
 * so the groups are frozen per chunk as described below and the window is
 * causal, which reduces to exact causal MLA when no group is condensed).
 * Query i of the chunk sits at absolute position t = chunk_start + i (its
 * absorbed query at q + i*q_tok_stride + h*576; H a multiple of 16, or 1,
 * 2, 4 or 8 as in mla_latent_attn_decode) and
 * attends to representatives [0, m) (all visible) and raw cache rows
 * [raw_begin, t] (causal, inclusive). Requires raw_begin <= chunk_start.
 * The groups a chunk sees are frozen before its window: with window w and
 * group size g the caller passes m = floor((chunk_start - w) / g) (0 when
 * chunk_start <= w) and raw_begin = m g, after condensing those groups with
 * the g queries that follow each one.
 *  o_latent [C, H, 512] contiguous, dtype o_dtype; lse [C, H] fp32, optional. */
int mla_latent_attn_prefill_chunk(const void* q, int32_t q_dtype, int64_t q_tok_stride,
                                  int64_t chunk_start, int32_t C, int32_t H,
                                  const lca_latent_t* reps, int64_t m,
                                  const lca_latent_t* raw, int64_t raw_begin, float sm_scale,
                                  void* o_latent, int32_t o_dtype, float* lse,
                                  hipStream_t stream);

/* mla_latent_attn_prefill_chunk for sequence `seq` of a paged cache (a
 * serving layout; the attention is that of mla_latent_attn_prefill_chunk,
 * 整体框架): query i of the chunk at position t = chunk_start + i attends
 * representatives [0, m) (dense packed bf16 rows, reps->c_tok_stride equal
 * to cache->row_stride; reps may be null when m = 0) and the cache tokens
 * [raw_begin, t] of sequence seq, token u at row u % page_rows of page
 * block_table[seq * table_stride + u / page_rows]. page_rows is a multiple
 * of 16. The caller guarantees that the block table maps every token in
 * [raw_begin, chunk_start + C) to a page of the pool (not checked). q,
 * o_latent, lse, dtypes and errors as in mla_latent_attn_prefill_chunk.
 * Tiles are formed as in the dense call, so on the same rows and
 * representatives the results are bitwise equal to it. */
int mla_latent_attn_prefill_chunk_paged(const void* q, int32_t q_dtype, int64_t q_tok_stride,
                                        int64_t chunk_start, int32_t C, int32_t H,
                                        const lca_latent_t* reps, int64_t m, const lca_paged_t* cache,
                                        int32_t seq, int64_t raw_begin, float sm_scale, void* o_latent,
                                        int32_t o_dtype, float* lse, hipStream_t stream);

/* mla_latent_attn_prefill_chunk and mla_latent_attn_prefill_chunk_paged with
 * a scheduling counter: the same attention (整体框架) and the same outputs,
 * bit for bit, computed by persistent workgroups (one per CU) that take the
 * chunk's query blocks (128 query rows each), heaviest first, from `sched`.
 * Workgroups are otherwise dealt to the XCDs by index, so a slower XCD would
 * end every chunk late; taken from one counter, the blocks go to whichever
 * workgroup is free. sched: device memory of two int32, 8-byte aligned,
 * owned by the caller; it must hold zeros before the first call, and every
 * call leaves zeros behind (the last workgroup resets it), so one pair
 * serves any number of calls in a stream or a replayed graph. Calls that can
 * run at the same time (other streams) need pairs of their own. The counter
 * is used by the packed-bf16 kernel; layouts that take the register-staged
 * kernel ignore it. Errors as in the calls above, and LCA_ERR_INVALID_ARG
 * for a null or misaligned sched. */
int mla_latent_attn_prefill_chunk_sched(const void* q, int32_t q_dtype, int64_t q_tok_stride,
                                        int64_t chunk_start, int32_t C, int32_t H,
                                        const lca_latent_t* reps, int64_t m,
                                        const lca_latent_t* raw, int64_t raw_begin, float sm_scale,
                                        void* o_latent, int32_t o_dtype, float* lse,
                                        int32_t* sched, hipStream_t stream);
int mla_latent_attn_prefill_chunk_paged_sched(const void* q, int32_t q_dtype, int64_t q_tok_stride,
                                              int64_t chunk_start, int32_t C, int32_t H,
                                              const lca_latent_t* reps, int64_t m, const lca_paged_t* cache,
                                              int32_t seq, int64_t raw_begin, float sm_scale, void* o_latent,
                                              int32_t o_dtype, float* lse, int32_t* sched, hipStream_t stream);

/* Per-head value up-projection (the MLA page's projection back to the head
 * space, 三.1): out[t, h, :] = o_latent[t, h, :] @ W_UV[h].
 *  o_latent [T, H, 512] contiguous (bf16 or f32); w_uv [H, 512, 128]
 *  contiguous (bf16 or f32); out [T, H, 128] contiguous, dtype out_dtype.
 *  bf16 matrix-core products with fp32 accumulation. T == 0 is a no-op. */
int mla_up_proj(const void* o_latent, int32_t o_dtype, int64_t T, int32_t H, const void* w_uv,
                int32_t w_dtype, void* out, int32_t out_dtype, hipStream_t stream);

/* Workspace bytes lca_project needs: the per-head no-RoPE query parts of the
 * T tokens, bf16 [T, H, 128]. */
size_t lca_project_workspace_size(int64_t T, int32_t H);

/* The projection step in front of the attention (MLA: "新一代开源大模型架构
 * 演进与注意力机制深度对比解析" 三.1, a per-token latent down-projection, with
 * RoPE handled apart; LCT page 研究背景与动机 / 核心矛盾: the position key K^R
 * beside the latent C^KV). For every token t with hidden state x_t and
 * position p_t = pos[t]:
 *   y = W x_t with W = w_proj, bf16 [576 + 192 H, d_model] row-major: row n
 *   holds the weights of output n. Outputs [0, 512) are c_t (W_DKV), [512,
 *   576) the RoPE key before rotation (W_KR), then for head h outputs
 *   576 + 192 h + [0, 128) are q^nope_h and + [128, 192) q^rope_h (W_Q).
 *   RoPE(v, p) rotates the 64-wide v in pairs (i, i + 32) by the angle
 *   p * rope_base^(-i / 32): (v_i, v_{i+32}) -> (v_i cos - v_{i+32} sin,
 *   v_{i+32} cos + v_i sin).
 * Writes
 *   the cache row [c_t ; RoPE(k_t, p_t)] (bf16, 576 values) at
 *     rows + dst_row[t] * row_stride, skipped where dst_row[t] < 0 (the
 *     append: dst_row is a device int64 [T] array of row indices into the
 *     caller's cache or page pool);
 *   the absorbed query of every head h at q + t * q_tok_stride + 576 h
 *     (dtype q_dtype): [W_UK[h] q^nope_h ; RoPE(q^rope_h, p_t)] with w_uk
 *     bf16 [H, 512, 128] (W_UK[h][j][k] multiplies q^nope_h[k]).
 * x is bf16 [T, d_model] with token stride x_tok_stride; pos is a device int32
 * [T] array. Matrix products run on bf16 operands with fp32 accumulation;
 * q^nope is rounded to bf16 before the W_UK product. d_model must be a
 * multiple of 32. The caller guarantees that the dst_row values name rows
 * inside its buffer and that no two tokens share one (not checked). q and
 * rows must not overlap any input. workspace >=
 * lca_project_workspace_size(T, H) bytes, 16-byte aligned; overwritten.
 * T == 0 is a no-op. */
int lca_project(const void* x, int64_t x_tok_stride, int64_t T, int32_t d_model, const int32_t* pos,
                double rope_base, const void* w_proj, const void* w_uk, int32_t H, void* rows,
                int64_t row_stride, const int64_t* dst_row, void* q, int32_t q_dtype, int64_t q_tok_stride,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LCA_H_ */
