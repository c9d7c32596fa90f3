// Per-head W_UV up-projection of a few rows (decode: one row per sequence),
// shared by mla_up_proj (rows read from o_latent) and the fused decode path
// (rows produced by merging the split partial results). Both sources go
// through the same kernel, so the two paths give bitwise equal outputs.
//
// MLA keeps only the latent per token and projects back to each head's value
// space at compute time ("新一代开源大模型架构演进与注意力机制深度对比解析",
// 三.1): out[t, h, :] = row[t, h, :] @ W_UV[h].
//
// Workgroup (2 rows, head h) of 4 wavefronts; the grid walks heads fastest,
// so with H a multiple of 8 every workgroup of head h lands on the same XCD
// and W_UV[h] (128 KB in bf16) is read from HBM about once per XCD and from
// that XCD's L2 afterwards. Wave w covers k in [128 w, 128 w + 128) as two
// 64-deep slices; lane (kg, col) holds 8 consecutive outputs of 8
// consecutive W rows and half-word shuffles turn them into the B operands of
// eight 16-output MFMA tiles (output n = 8 col + c). Each slice is a chain of
// two 16x16x32 MFMA; the 8 slice partials are added in slice order.
#pragma once
#include "lca.h"
#include "lca_device.h"
#include "lca_internal.h"

#include <type_traits>

namespace lca {

constexpr int UPR_TOK = 2;     // rows per workgroup
constexpr int UPR_WAVES = 4;   // wavefronts per workgroup
constexpr int UPR_SLICES = 8;  // 64-deep k slices, summed in order

// ---- split-K merge of decode partials
constexpr int MERGE_SMALL_S = 32;
constexpr int MERGE_BATCH = 8;  // split outputs loaded together

// Merged columns [4 c4, 4 c4 + 4) of one (sequence, head) from S split
// partials (slot(s) = (slot0 + s) * 16 + hh; ml = running max (log2 units)
// and sum, o = unnormalised output), and the merged max M and sum L:
//   o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s,
// always in split order. Every load of a batch is issued before any is
// used, so the merge is one or two memory round trips long.
__device__ __forceinline__ float4 merge_cols4(const float* __restrict__ part_o,
                                              const float* __restrict__ part_ml, int S,
                                              int64_t slot0, int hh, int c4, float& M, float& L) {
  const float2* ml = reinterpret_cast<const float2*>(part_ml);
  const float4* po = reinterpret_cast<const float4*>(part_o);
  float2 v_ml[MERGE_SMALL_S];
#pragma unroll
  for (int s = 0; s < MERGE_SMALL_S; ++s)
    v_ml[s] = s < S ? ml[(slot0 + s) * HB + hh] : make_float2(-INFINITY, 0.f);
  float4 v_o[MERGE_BATCH];
#pragma unroll
  for (int s = 0; s < MERGE_BATCH; ++s)
    v_o[s] = s < S ? po[((slot0 + s) * HB + hh) * (D_C / 4) + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
  M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MERGE_SMALL_S; ++s) M = fmaxf(M, v_ml[s].x);
  L = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s0 = 0; s0 < MERGE_SMALL_S; s0 += MERGE_BATCH) {
    if (s0 >= S) break;
    if (s0 > 0) {
#pragma unroll
      for (int s = 0; s < MERGE_BATCH; ++s)
        v_o[s] = s0 + s < S ? po[((slot0 + s0 + s) * HB + hh) * (D_C / 4) + c4]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int s = 0; s < MERGE_BATCH; ++s) {
      const float ms = v_ml[s0 + s].x;
      const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
      L = fmaf(wgt, v_ml[s0 + s].y, L);
      a.x = fmaf(wgt, v_o[s].x, a.x); a.y = fmaf(wgt, v_o[s].y, a.y);
      a.z = fmaf(wgt, v_o[s].z, a.z); a.w = fmaf(wgt, v_o[s].w, a.w);
    }
  }
  const float inv = 1.0f / L;
  return make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
}

// The same merge in two steps for S <= MERGE_BATCH: every load first
// (merge_load), the arithmetic later (merge_math), so that a kernel can put
// other loads in flight between them. The loads take no branch (a branch per
// load made the compiler wait for each one); merge_math masks the splits past
// S. The arithmetic is merge_cols4's, in the same order, so the two give
// bitwise equal results.
struct MergeLoads {
  float2 ml[MERGE_BATCH];
  float4 o[MERGE_BATCH];
};
__device__ __forceinline__ void merge_load(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                           int S, int64_t slot0, int hh, int c4, MergeLoads& ld) {
  const float2* ml = reinterpret_cast<const float2*>(part_ml);
  const float4* po = reinterpret_cast<const float4*>(part_o);
#pragma unroll
  for (int s = 0; s < MERGE_BATCH; ++s) {  // splits past S reload split S - 1 (no branch per load)
    const int64_t sl = slot0 + (s < S ? s : S - 1);
    ld.ml[s] = ml[sl * HB + hh];
    ld.o[s] = po[(sl * HB + hh) * (D_C / 4) + c4];
  }
}
__device__ __forceinline__ float4 merge_math(const MergeLoads& ld, int S, float& M, float& L) {
  float2 v_ml[MERGE_BATCH];
  float4 v_o[MERGE_BATCH];
#pragma unroll
  for (int s = 0; s < MERGE_BATCH; ++s) {
    v_ml[s] = s < S ? ld.ml[s] : make_float2(-INFINITY, 0.f);
    v_o[s] = s < S ? ld.o[s] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MERGE_BATCH; ++s) M = fmaxf(M, v_ml[s].x);
  L = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < MERGE_BATCH; ++s) {
    const float ms = v_ml[s].x;
    const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
    L = fmaf(wgt, v_ml[s].y, L);
    a.x = fmaf(wgt, v_o[s].x, a.x); a.y = fmaf(wgt, v_o[s].y, a.y);
    a.z = fmaf(wgt, v_o[s].z, a.z); a.w = fmaf(wgt, v_o[s].w, a.w);
  }
  const float inv = 1.0f / L;
  return make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
}

// ---- row sources
// A source's loads can be issued (prefetch) before its arithmetic (finish).
template <typename TO>
struct RowsFromLatent {  // o_latent [T, H, 512]
  const TO* x;
  typedef float4 Pre;
  __device__ __forceinline__ void prefetch(int64_t t, int h, int H, int c4, Pre& v) const {
    const TO* p = x + (t * H + h) * D_C + 4 * c4;
    v = make_float4(to_f32(p[0]), to_f32(p[1]), to_f32(p[2]), to_f32(p[3]));
  }
  __device__ __forceinline__ float4 finish(const Pre& v, int64_t, int, int, int) const { return v; }
};
template <>
struct RowsFromLatent<float> {
  const float* x;
  typedef float4 Pre;
  __device__ __forceinline__ void prefetch(int64_t t, int h, int H, int c4, Pre& v) const {
    v = reinterpret_cast<const float4*>(x + (t * H + h) * D_C)[c4];
  }
  __device__ __forceinline__ float4 finish(const Pre& v, int64_t, int, int, int) const { return v; }
};

struct RowsFromSplits {  // decode partials; writes o_latent and lse as it merges
  const float* part_o;
  const float* part_ml;
  int S;
  float* o;
  float* lse;
  typedef MergeLoads Pre;  // the loads of a merge over at most MERGE_BATCH splits
  __device__ __forceinline__ void prefetch(int64_t b, int h, int H, int c4, Pre& ld) const {
    if (S <= MERGE_BATCH) {  // uniform
      const int HG = head_blocks(H), hg = h / HB, hh = h % HB;
      merge_load(part_o, part_ml, S, (b * HG + hg) * S, hh, c4, ld);
    }
  }
  __device__ __forceinline__ float4 finish(const Pre& ld, int64_t b, int h, int H, int c4) const {
    const int HG = head_blocks(H), hg = h / HB, hh = h % HB;
    float M, L;
    const float4 v = S <= MERGE_BATCH ? merge_math(ld, S, M, L)
                                      : merge_cols4(part_o, part_ml, S, (b * HG + hg) * S, hh, c4, M, L);
    reinterpret_cast<float4*>(o + (b * H + h) * D_C)[c4] = v;
    if (lse != nullptr && c4 == 0) lse[b * H + h] = (M + log2f(L)) * 0.69314718055994530942f;
    return v;
  }
};

// No extra work after the up-projection blocks.
struct NoStep {
  int B = 0;
  __device__ void run(int) const {}
};

// Grid: ceil(T / UPR_TOK) * H up-projection workgroups, then step.B
// workgroups that run step.run(b) for b < step.B (work that must follow the
// previous kernel, appended here instead of launched on its own).
template <class Src, typename TW, typename TY, class Step = NoStep>
__global__ __launch_bounds__(64 * UPR_WAVES) void up_rows_kernel(Src src, int64_t T, int H,
                                                                 const TW* __restrict__ wuv,
                                                                 TY* __restrict__ y, Step step = Step{}) {
  if constexpr (!std::is_same<Step, NoStep>::value) {
    const int64_t n_up = ((T + UPR_TOK - 1) / UPR_TOK) * H;
    if ((int64_t)blockIdx.x >= n_up) {  // workgroup-uniform
      step.run((int)((int64_t)blockIdx.x - n_up));
      return;
    }
  }
  __shared__ __align__(16) bf16_t rows[UPR_TOK][D_C + 8];
  __shared__ __align__(16) float red[UPR_SLICES][UPR_TOK][D_V + 4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int h = (int)(blockIdx.x % (unsigned)H);
  const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)H) * UPR_TOK;

  // the rows' loads first (thread -> row ri, columns 4 rc4 .. 4 rc4 + 3):
  // a merge of split partials is on this kernel's critical path, W_UV is not
  const int ri = tid / (D_C / 4), rc4 = tid % (D_C / 4);
  const int64_t rt = t0 + ri;
  const bool has_row = ri < UPR_TOK && rt < T;
  typename Src::Pre pre;
  if (has_row) src.prefetch(rt, h, H, rc4, pre);
  __builtin_amdgcn_sched_barrier(0);

  // W_UV[h] rows 128 w + 32 ks + 8 kg + kk, outputs 8 col .. 8 col + 7
  const TW* wh = wuv + (int64_t)h * D_C * D_V + 8 * col;
  uint4 R[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      R[ks][kk] = raw8_bf16(raw8_load(wh + (int64_t)(128 * w + 32 * ks + 8 * kg + kk) * D_V));

  {  // the rows, as bf16 A-operand source
    uint2 packed = make_uint2(0u, 0u);
    if (has_row) {
      const float4 v = src.finish(pre, rt, h, H, rc4);
      packed = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
    }
    if (ri < UPR_TOK) *reinterpret_cast<uint2*>(&rows[ri][4 * rc4]) = packed;
  }
  __syncthreads();

  uint4 a[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    a[ks] = col < UPR_TOK ? *reinterpret_cast<const uint4*>(&rows[col][128 * w + 32 * ks + 8 * kg])
                          : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // slice 2 w + j: k in [128 w + 64 j, + 64)
    f32x4_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int wi = c >> 1;
      uint4 bop[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ks = 2 * j + q;
        uint32_t r[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) r[kk] = u4_get(R[ks][kk], wi);
        bop[q] = (c & 1) ? make_uint4(hi_pair(r[0], r[1]), hi_pair(r[2], r[3]), hi_pair(r[4], r[5]), hi_pair(r[6], r[7]))
                         : make_uint4(lo_pair(r[0], r[1]), lo_pair(r[2], r[3]), lo_pair(r[4], r[5]), lo_pair(r[6], r[7]));
      }
      acc[c] = mfma16x16x32(a[2 * j], bop[0], f32x4_t{0.f, 0.f, 0.f, 0.f});
      acc[c] = mfma16x16x32(a[2 * j + 1], bop[1], acc[c]);
    }
    // acc[c][r] = slice partial of out[row 4 kg + r][8 col + c]; rows >= UPR_TOK are padding
    if (kg == 0) {
#pragma unroll
      for (int r = 0; r < UPR_TOK; ++r) {
        float* dst = &red[2 * w + j][r][8 * col];
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
      }
    }
  }
  __syncthreads();
  if (tid < UPR_TOK * (D_V / 4)) {  // thread -> (row, 4 outputs); slices added in order
    const int i = tid / (D_V / 4), c4 = tid % (D_V / 4);
    const int64_t t = t0 + i;
    if (t < T) {
      float4 v = *reinterpret_cast<const float4*>(&red[0][i][4 * c4]);
#pragma unroll
      for (int s = 1; s < UPR_SLICES; ++s) {
        const float4 u = *reinterpret_cast<const float4*>(&red[s][i][4 * c4]);
        v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
      }
      TY* yp = y + (t * H + h) * D_V + 4 * c4;
      yp[0] = from_f32<TY>(v.x); yp[1] = from_f32<TY>(v.y);
      yp[2] = from_f32<TY>(v.z); yp[3] = from_f32<TY>(v.w);
    }
  }
}

template <class Src, typename TW>
inline void launch_up_rows(const Src& src, int64_t T, int H, const void* w_uv, void* out,
                           int out_dtype, hipStream_t stream) {
  const dim3 grid((unsigned)(((T + UPR_TOK - 1) / UPR_TOK) * H));
  if (out_dtype == LCA_BF16)
    hipLaunchKernelGGL((up_rows_kernel<Src, TW, bf16_t>), grid, dim3(64 * UPR_WAVES), 0, stream, src, T, H,
                       (const TW*)w_uv, (bf16_t*)out);
  else
    hipLaunchKernelGGL((up_rows_kernel<Src, TW, float>), grid, dim3(64 * UPR_WAVES), 0, stream, src, T, H,
                       (const TW*)w_uv, (float*)out);
}

}  // namespace lca
