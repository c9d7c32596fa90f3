// Launchers shared between the host API (lca_api.cpp) and the kernel files.
// Arguments are already validated when these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lca.h"

namespace lca {

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
                                 float sm_scale, const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq,
                                 float* alpha, int64_t alpha_seq, float* qbar_ws, hipStream_t stream);
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

// decode followed by the W_UV up-projection of its output; the split merge
// and the projection share one kernel when B <= UP_SMALL_T.
hipError_t launch_decode_paged(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                               const lca_latent_t& reps, const int32_t* seq_m, const lca_paged_t& cache,
                               const int32_t* seq_raw_begin, const int32_t* seq_raw_end,
                               int64_t max_entries, float sm_scale, float* o_latent, float* lse,
                               void* workspace, hipStream_t stream);
hipError_t launch_decode_up(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                            const lca_latent_t& reps, int64_t m, const lca_latent_t& raw,
                            int64_t raw_begin, int64_t raw_end, float sm_scale, float* o_latent,
                            float* lse, const void* w_uv, int w_dtype, void* out, int out_dtype,
                            void* workspace, hipStream_t stream);

// ---- prefill
hipError_t launch_prefill(const void* q, int q_dtype, int64_t q_tok_stride, int64_t chunk_start,
                          int C, int H, const lca_latent_t& reps, int64_t m,
                          const lca_latent_t& raw, int64_t raw_begin, float sm_scale,
                          void* o_latent, int o_dtype, float* lse, hipStream_t stream);

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
