// Launchers shared between the host API (lca_api.cpp) and the kernel files.
// Arguments are already validated when these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lca.h"

namespace lca {

// Head counts: the attention kernels work on blocks of 16 heads (one side of
// a 16-row matrix tile). H may be a multiple of 16, or a divisor of 16 (a
// grouped-query attention group of 1, 2, 4 or 8 heads, held in one block
// whose rows past H repeat a valid query and are never stored).
constexpr int HEAD_BLOCK = 16;
__host__ __device__ inline bool heads_supported(int H) { return H >= 1 && (H % HEAD_BLOCK == 0 || HEAD_BLOCK % H == 0); }
__host__ __device__ inline int head_blocks(int H) { return (H + HEAD_BLOCK - 1) / HEAD_BLOCK; }

struct Seg {  // one latent tensor segment, strides in elements
  const void* c;
  const void* kr;
  int64_t c_seq, c_tok, kr_seq, kr_tok;
};

inline Seg to_seg(const lca_latent_t& t) {
  return Seg{t.c, t.kr, t.c_seq_stride, t.c_tok_stride, t.kr_seq_stride, t.kr_tok_stride};
}

// ---- condensation
hipError_t launch_condense_paged(const lca_paged_t& cache, int B, int g, const int32_t* seq_group_begin,
                                 const int32_t* seq_n_groups, int64_t max_groups, const void* q, int q_dtype,
                                 int64_t q_seq_stride, int64_t q_tok_stride, int H, int64_t q_row0,
                                 int64_t q_row_step, float sm_scale, const lca_latent_t& reps, int32_t* anchor,
                                 int64_t anchor_seq, float* alpha, int64_t alpha_seq, float* qbar_ws,
                                 hipStream_t stream);
// one decode step's incremental condensation and state update (paged cache)
hipError_t launch_condense_step(const lca_paged_t& cache, int B, int64_t w, int g, const void* q, int q_dtype,
                                int64_t q_seq_stride, int H, void* q_ring, int64_t q_ring_seq_stride,
                                float sm_scale, const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq,
                                int32_t* seq_m, int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos,
                                int64_t* dst_row, hipStream_t stream);
// the W_UV up-projection of a decode's rows (up_rows_kernel: merging the S > 1
// split partials, or over the merged fp32 o_latent when S = 1) with the step
// condensation appended as B workgroups of the same launch (B <= UP_SMALL_T)
hipError_t launch_up_rows_step(const float* part_o, const float* part_ml, int S, float* o_latent, float* lse,
                               int B, int H, const void* w_uv, int w_dtype, void* out, int out_dtype,
                               const lca_paged_t& cache, int64_t w, int g, const void* q, int q_dtype,
                               int64_t q_seq_stride, void* q_ring, int64_t q_ring_seq_stride, float sm_scale,
                               const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq, int32_t* seq_m,
                               int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos, int64_t* dst_row,
                               hipStream_t stream);
hipError_t launch_condense(const lca_latent_t& cache, int B, int g, int64_t group_begin,
                           int64_t n_groups, const void* q, int q_dtype, int64_t q_seq_stride,
                           int64_t q_tok_stride, int H, int64_t q_row0, int64_t q_row_step,
                           float sm_scale, const lca_latent_t& reps, int32_t* anchor,
                           int64_t anchor_seq, float* alpha, int64_t alpha_seq, float* qbar_ws,
                           int mode, hipStream_t stream);

// ---- decode
constexpr int QBAR_PARTS = 8;            // partial sums per shared summary query
constexpr int DEC_TARGET_BLOCKS = 256;   // split-K aims for about one workgroup per CU

struct DecodeSplit {
  int S;         // splits per (sequence, head block)
  int per_tiles; // tiles per split
};
DecodeSplit decode_split(int B, int HG, int64_t n_entries);
size_t decode_workspace_bytes(int B, int HG, int S);

hipError_t launch_decode(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                         const lca_latent_t& reps, int64_t m, const lca_latent_t& raw,
                         int64_t raw_begin, int64_t raw_end, float sm_scale, float* o_latent,
                         float* lse, void* workspace, hipStream_t stream);

// Scratch of the entry point that allocates nothing: a file-scope device
// array of NOALLOC_SCRATCH_BYTES (every split plan of decode_split fits), its
// device address for the current device (looked up once per device).
constexpr size_t NOALLOC_SCRATCH_BYTES = LCA_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** out);

// decode followed by the W_UV up-projection of its output; the split merge
// and the projection share one kernel when B <= UP_SMALL_T.
hipError_t launch_decode_paged(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                               const lca_latent_t& reps, const int32_t* seq_m, const lca_paged_t& cache,
                               const int32_t* seq_raw_begin, const int32_t* seq_raw_end,
                               int64_t max_entries, float sm_scale, float* o_latent, float* lse,
                               void* workspace, hipStream_t stream);
hipError_t launch_decode_paged_up(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                                  const lca_latent_t& reps, const int32_t* seq_m, const lca_paged_t& cache,
                                  const int32_t* seq_raw_begin, const int32_t* seq_raw_end, int64_t max_entries,
                                  float sm_scale, float* o_latent, float* lse, const void* w_uv, int w_dtype,
                                  void* out, int out_dtype, void* workspace, hipStream_t stream);
// launch_decode_paged_up followed by the step condensation (lca_condense_step),
// the latter inside the merge/up-projection launch when that kernel runs
hipError_t launch_decode_paged_up_step(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                                       const lca_latent_t& reps, int32_t* seq_m, const lca_paged_t& cache,
                                       int32_t* seq_raw_begin, int32_t* seq_raw_end, int64_t max_entries,
                                       float sm_scale, float* o_latent, float* lse, const void* w_uv, int w_dtype,
                                       void* out, int out_dtype, void* workspace, int64_t w, int g, void* q_ring,
                                       int64_t q_ring_seq_stride, int32_t* anchor, int64_t anchor_seq, int32_t* pos,
                                       int64_t* dst_row, hipStream_t stream);
hipError_t launch_decode_up(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                            const lca_latent_t& reps, int64_t m, const lca_latent_t& raw,
                            int64_t raw_begin, int64_t raw_end, float sm_scale, float* o_latent,
                            float* lse, const void* w_uv, int w_dtype, void* out, int out_dtype,
                            void* workspace, hipStream_t stream);

// ---- prefill
hipError_t launch_prefill(const void* q, int q_dtype, int64_t q_tok_stride, int64_t chunk_start,
                          int C, int H, const lca_latent_t& reps, int64_t m,
                          const lca_latent_t& raw, int64_t raw_begin, float sm_scale,
                          void* o_latent, int o_dtype, float* lse, hipStream_t stream,
                          int* sched = nullptr);

// chunked prefill of sequence `seq` of a paged cache (raw rows through its
// block table; representatives dense, same row stride as the pages). With
// sched (two ints, zero on entry, zero again when the launch ends) the
// packed-row kernel runs as persistent workgroups taking blocks from it.
hipError_t launch_prefill_paged(const void* q, int q_dtype, int64_t q_tok_stride, int64_t chunk_start,
                                int C, int H, const lca_latent_t& reps, int64_t m, const lca_paged_t& cache,
                                int seq, int64_t raw_begin, float sm_scale, void* o_latent, int o_dtype,
                                float* lse, hipStream_t stream, int* sched = nullptr);

// ---- up-projection
constexpr int UP_SMALL_T = 64;  // token counts up to this use the small-T kernel
hipError_t launch_up_proj(const void* o_latent, int o_dtype, int64_t T, int H, const void* w_uv,
                          int w_dtype, void* out, int out_dtype, hipStream_t stream);

// ---- projection step (hidden states -> cache rows and absorbed queries)
hipError_t launch_project(const void* x, int64_t x_stride, int64_t T, int d, const int32_t* pos,
                          double rope_base, const void* w_proj, const void* w_uk, int H, void* rows,
                          int64_t row_stride, const int64_t* dst_row, void* q, int q_dtype,
                          int64_t q_stride, void* qn, hipStream_t stream);

}  // namespace lca
