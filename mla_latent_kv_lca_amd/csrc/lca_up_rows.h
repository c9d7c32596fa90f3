// Per-head W_UV up-projection of a few rows (decode: one row per sequence),
// shared by mla_up_proj (rows read from o_latent) and the fused decode path
// (rows produced by merging the split partial results). Both sources go
// through the same kernel, so the two paths give bitwise equal outputs.
//
// MLA keeps only the latent per token and projects back to each head's value
// space at compute time ("新一代开源大模型架构演进与注意力机制深度对比解析",
// 三.1): out[t, h, :] = row[t, h, :] @ W_UV[h].
//
// Workgroup (R rows, head h, a block of 128 / F output columns) of 4
// wavefronts; the grid walks heads fastest, so with H a multiple of 8 every
// workgroup of head h lands on the same XCD and W_UV[h] (128 KB in bf16) is
// read from HBM about once per XCD and from that XCD's L2 afterwards. The
// kernel is bound by the bytes each workgroup pulls through its CU (W_UV's
// column block plus its rows), so the host picks R and F per call: few rows
// with many splits each take one row and half the columns, a batch of 32
// merged 8-split rows four rows and half the columns, a single row an eighth
// of the columns.
#pragma once
#include "lca.h"
#include "lca_device.h"
#include "lca_internal.h"

#include <type_traits>

namespace lca {

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
  // per-lane bases plus a wave-uniform offset per split, so that each load
  // costs one address add
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + slot0 * HB + hh;
  const float4* po = reinterpret_cast<const float4*>(part_o) + (slot0 * HB + hh) * (D_C / 4) + c4;
#pragma unroll
  for (int s = 0; s < MERGE_BATCH; ++s) {  // splits past S reload split S - 1 (no branch per load)
    const int sc = s < S ? s : S - 1;
    ld.ml[s] = ml[(int64_t)sc * HB];
    ld.o[s] = po[(int64_t)sc * HB * (D_C / 4)];
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
// finish(..., store) also writes whatever the source produces besides the
// row (the merged o_latent and lse) when store is set. On the host,
// row_bytes() is what one row costs to fetch and four_rows() whether a thread
// may hold the loads of two rows at once.
template <typename TO>
struct RowsFromLatent {  // o_latent [T, H, 512]
  const TO* x;
  typedef float4 Pre;
  __device__ __forceinline__ void prefetch(int64_t t, int h, int H, int c4, Pre& v) const {
    const TO* p = x + (t * H + h) * D_C + 4 * c4;
    v = make_float4(to_f32(p[0]), to_f32(p[1]), to_f32(p[2]), to_f32(p[3]));
  }
  __device__ __forceinline__ float4 finish(const Pre& v, int64_t, int, int, int, bool) const { return v; }
  int64_t row_bytes() const { return (int64_t)D_C * sizeof(TO); }
  bool four_rows() const { return true; }
};
template <>
struct RowsFromLatent<float> {
  const float* x;
  typedef float4 Pre;
  __device__ __forceinline__ void prefetch(int64_t t, int h, int H, int c4, Pre& v) const {
    v = reinterpret_cast<const float4*>(x + (t * H + h) * D_C)[c4];
  }
  __device__ __forceinline__ float4 finish(const Pre& v, int64_t, int, int, int, bool) const { return v; }
  int64_t row_bytes() const { return (int64_t)D_C * sizeof(float); }
  bool four_rows() const { return true; }
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
  __device__ __forceinline__ float4 finish(const Pre& ld, int64_t b, int h, int H, int c4, bool store) const {
    const int HG = head_blocks(H), hg = h / HB, hh = h % HB;
    float M, L;
    const float4 v = S <= MERGE_BATCH ? merge_math(ld, S, M, L)
                                      : merge_cols4(part_o, part_ml, S, (b * HG + hg) * S, hh, c4, M, L);
    if (store) {
      reinterpret_cast<float4*>(o + (b * H + h) * D_C)[c4] = v;
      if (lse != nullptr && c4 == 0) lse[b * H + h] = (M + log2f(L)) * 0.69314718055994530942f;
    }
    return v;
  }
  int64_t row_bytes() const { return (int64_t)S * (D_C + 2) * (int64_t)sizeof(float); }
  bool four_rows() const { return false; }  // two merges per thread: measured slower than two rows per workgroup
};

// No extra work after the up-projection blocks.
struct NoStep {
  int B = 0;
  __device__ void run(int) const {}
};

// CT consecutive W_UV outputs of one row as packed bf16: element c in half
// c & 1 of word c >> 1 (CT = 1: the low half of one word).
template <int CT>
struct WFrag {
  uint32_t u[(CT + 1) / 2];
};
template <int CT>
__device__ __forceinline__ WFrag<CT> wfrag_load(const bf16_t* p) {
  WFrag<CT> f;
  if constexpr (CT == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    f.u[0] = v.x; f.u[1] = v.y; f.u[2] = v.z; f.u[3] = v.w;
  } else if constexpr (CT == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    f.u[0] = v.x; f.u[1] = v.y;
  } else if constexpr (CT == 2) {
    f.u[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    f.u[0] = (uint32_t)*reinterpret_cast<const uint16_t*>(p);
  }
  return f;
}
template <int CT>
__device__ __forceinline__ WFrag<CT> wfrag_load(const float* p) {
  WFrag<CT> f;
  if constexpr (CT == 8) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    f.u[0] = pack_bf2(a.x, a.y); f.u[1] = pack_bf2(a.z, a.w);
    f.u[2] = pack_bf2(b.x, b.y); f.u[3] = pack_bf2(b.z, b.w);
  } else if constexpr (CT == 4) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    f.u[0] = pack_bf2(a.x, a.y); f.u[1] = pack_bf2(a.z, a.w);
  } else if constexpr (CT == 2) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    f.u[0] = pack_bf2(a.x, a.y);
  } else {
    f.u[0] = f2bf(*p);
  }
  return f;
}

// Workgroup shape of up_rows_kernel: R rows of one head, output columns
// [fb NC, fb NC + NC) of F blocks (NC = 128 / F), always 4 wavefronts.
template <int R_, int F_>
struct UpShape {
  static constexpr int R = R_;          // rows (1, 2 or 4)
  static constexpr int F = F_;          // output-column blocks per head (1, 2 or 8)
  static constexpr int NC = D_V / F_;   // output columns per workgroup
  static constexpr int CT = NC / 16;    // 16-output MFMA tiles = outputs per lane
  static constexpr int RPT = R_ > 2 ? 2 : 1;  // rows merged per thread
  static_assert(R_ == 1 || R_ == 2 || R_ == 4, "rows per workgroup");
  static_assert(CT >= 1 && CT <= 8 && NC == 16 * CT, "column blocks");
};
typedef UpShape<2, 1> UpShapeStep;  // the shape of launches that carry step workgroups

// Grid: ceil(T / R) * H * F up-projection workgroups (head fastest, then
// column block, then row group), then step.B workgroups that run
// step.run(b) for b < step.B (work that must follow the previous kernel,
// appended here instead of launched on its own).
//
// Wave w covers k in [128 w, 128 w + 128) as two 64-deep slices; lane (kg,
// col) holds CT consecutive outputs (CT col .. CT col + CT - 1 of the
// workgroup's block) of 8 consecutive W rows per 32-deep step, and half-word
// shuffles turn them into the B operands of CT 16-output MFMA tiles (tile c
// holds outputs CT col' + c). Each slice is a chain of two 16x16x32 MFMA; the
// 8 slice partials are added in slice order. An output's arithmetic is the
// same in every shape, so the shapes give bitwise equal results.
template <class Src, typename TW, typename TY, class Step = NoStep, class Sh = UpShapeStep>
__global__ __launch_bounds__(64 * UPR_WAVES) void up_rows_kernel(Src src, int64_t T, int H,
                                                                 const TW* __restrict__ wuv,
                                                                 TY* __restrict__ y, Step step = Step{}) {
  constexpr int R = Sh::R, F = Sh::F, NC = Sh::NC, CT = Sh::CT, RPT = Sh::RPT;
  if constexpr (!std::is_same<Step, NoStep>::value) {
    const int64_t n_up = ((T + R - 1) / R) * H * F;
    if ((int64_t)blockIdx.x >= n_up) {  // workgroup-uniform
      step.run((int)((int64_t)blockIdx.x - n_up));
      return;
    }
  }
  __shared__ __align__(16) bf16_t rows[R][D_C + 8];
  __shared__ __align__(16) float red[UPR_SLICES][R][NC + 4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int h = (int)(blockIdx.x % (unsigned)H);
  const unsigned rest = blockIdx.x / (unsigned)H;
  const int fb = (int)(rest % (unsigned)F);
  const int64_t t0 = (int64_t)(rest / (unsigned)F) * R;

  // the rows' loads first (thread -> rows ri + 2 p, columns 4 rc4 .. 4 rc4 +
  // 3): a merge of split partials is on this kernel's critical path, W_UV is
  // not
  const int ri = tid / (D_C / 4), rc4 = tid % (D_C / 4);
  const int64_t rt0 = t0 + ri, rt1 = rt0 + 2;
  const bool has0 = ri < R && rt0 < T, has1 = RPT > 1 && ri + 2 < R && rt1 < T;
  typename Src::Pre pre0, pre1;
  if (has0) src.prefetch(rt0, h, H, rc4, pre0);
  if constexpr (RPT > 1) {
    if (has1) src.prefetch(rt1, h, H, rc4, pre1);
  }
  __builtin_amdgcn_sched_barrier(0);

  // W_UV[h] rows 128 w + 32 ks + 8 kg + kk, block outputs CT col .. + CT - 1
  const TW* wh = wuv + (int64_t)h * D_C * D_V + NC * fb + CT * col;
  WFrag<CT> Wr[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      Wr[ks][kk] = wfrag_load<CT>(wh + (int64_t)(128 * w + 32 * ks + 8 * kg + kk) * D_V);

  {  // the rows, as bf16 A-operand source
    uint2 packed = make_uint2(0u, 0u);
    if (has0) {
      const float4 v = src.finish(pre0, rt0, h, H, rc4, fb == 0);
      packed = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
    }
    if (ri < R) *reinterpret_cast<uint2*>(&rows[ri][4 * rc4]) = packed;
  }
  if constexpr (RPT > 1) {
    uint2 packed = make_uint2(0u, 0u);
    if (has1) {
      const float4 v = src.finish(pre1, rt1, h, H, rc4, fb == 0);
      packed = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
    }
    if (ri + 2 < R) *reinterpret_cast<uint2*>(&rows[ri + 2][4 * rc4]) = packed;
  }
  __syncthreads();

  uint4 a[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    a[ks] = col < R ? *reinterpret_cast<const uint4*>(&rows[col][128 * w + 32 * ks + 8 * kg])
                    : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // slice 2 w + j: k in [128 w + 64 j, + 64)
    f32x4_t acc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int wi = c >> 1;
      uint4 bop[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ks = 2 * j + q;
        uint32_t r[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) r[kk] = Wr[ks][kk].u[wi];
        bop[q] = (c & 1) ? make_uint4(hi_pair(r[0], r[1]), hi_pair(r[2], r[3]), hi_pair(r[4], r[5]), hi_pair(r[6], r[7]))
                         : make_uint4(lo_pair(r[0], r[1]), lo_pair(r[2], r[3]), lo_pair(r[4], r[5]), lo_pair(r[6], r[7]));
      }
      acc[c] = mfma16x16x32(a[2 * j], bop[0], f32x4_t{0.f, 0.f, 0.f, 0.f});
      acc[c] = mfma16x16x32(a[2 * j + 1], bop[1], acc[c]);
    }
    // acc[c][r] = slice partial of out[row 4 kg + r][block output CT col + c];
    // rows >= R are padding
    if (kg == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float* dst = &red[2 * w + j][r][CT * col];
        if constexpr (CT >= 4) {
#pragma unroll
          for (int c = 0; c < CT; c += 4)
            *reinterpret_cast<float4*>(dst + c) = make_float4(acc[c][r], acc[c + 1][r], acc[c + 2][r], acc[c + 3][r]);
        } else {
#pragma unroll
          for (int c = 0; c < CT; ++c) dst[c] = acc[c][r];
        }
      }
    }
  }
  __syncthreads();
  if (tid < R * (NC / 4)) {  // thread -> (row, 4 outputs); slices added in order
    const int i = tid / (NC / 4), c4 = tid % (NC / 4);
    const int64_t t = t0 + i;
    if (t < T) {
      float4 v = *reinterpret_cast<const float4*>(&red[0][i][4 * c4]);
#pragma unroll
      for (int s = 1; s < UPR_SLICES; ++s) {
        const float4 u = *reinterpret_cast<const float4*>(&red[s][i][4 * c4]);
        v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
      }
      TY* yp = y + (t * H + h) * D_V + NC * fb + 4 * c4;
      yp[0] = from_f32<TY>(v.x); yp[1] = from_f32<TY>(v.y);
      yp[2] = from_f32<TY>(v.z); yp[3] = from_f32<TY>(v.w);
    }
  }
}

// The shape for T rows of H heads: by the bytes each workgroup pulls through
// its CU (W_UV[h]'s column block plus its rows, the bound of this kernel),
// scaled by how many workgroups share a CU when there are more than 256.
enum UpShapeId { UP_R2F1 = 0, UP_R1F2, UP_R1F8, UP_R4F1, UP_R4F2 };
inline UpShapeId up_rows_shape(int64_t T, int H, int64_t row_bytes, int64_t w_head_bytes, bool four_rows) {
  static const struct { UpShapeId id; int R, F; } cand[] = {
      {UP_R2F1, 2, 1}, {UP_R1F2, 1, 2}, {UP_R1F8, 1, 8}, {UP_R4F1, 4, 1}, {UP_R4F2, 4, 2}};
  UpShapeId best = UP_R2F1;
  double best_cost = 0.0;
  for (const auto& c : cand) {
    if (c.R == 4 && !four_rows) continue;
    const double wgs = (double)((T + c.R - 1) / c.R) * H * c.F;
    const double per_wg = (double)w_head_bytes / c.F + (double)c.R * row_bytes;
    const double cost = per_wg * (wgs > 256.0 ? wgs / 256.0 : 1.0);
    if (c.id == UP_R2F1 || cost < best_cost) {
      best = c.id;
      best_cost = cost;
    }
  }
  return best;
}

template <class Src, typename TW, typename TY, class Sh>
inline void launch_up_rows_shape(const Src& src, int64_t T, int H, const void* w_uv, void* out, hipStream_t stream) {
  const dim3 grid((unsigned)(((T + Sh::R - 1) / Sh::R) * H * Sh::F));
  hipLaunchKernelGGL((up_rows_kernel<Src, TW, TY, NoStep, Sh>), grid, dim3(64 * UPR_WAVES), 0, stream, src, T, H,
                     (const TW*)w_uv, (TY*)out, NoStep{});
}
template <class Src, typename TW, typename TY>
inline void launch_up_rows_typed(const Src& src, int64_t T, int H, const void* w_uv, void* out, hipStream_t stream) {
  switch (up_rows_shape(T, H, src.row_bytes(), (int64_t)D_C * D_V * sizeof(TW), src.four_rows())) {
    case UP_R1F2: launch_up_rows_shape<Src, TW, TY, UpShape<1, 2>>(src, T, H, w_uv, out, stream); break;
    case UP_R1F8: launch_up_rows_shape<Src, TW, TY, UpShape<1, 8>>(src, T, H, w_uv, out, stream); break;
    case UP_R4F1: launch_up_rows_shape<Src, TW, TY, UpShape<4, 1>>(src, T, H, w_uv, out, stream); break;
    case UP_R4F2: launch_up_rows_shape<Src, TW, TY, UpShape<4, 2>>(src, T, H, w_uv, out, stream); break;
    default: launch_up_rows_shape<Src, TW, TY, UpShape<2, 1>>(src, T, H, w_uv, out, stream); break;
  }
}
template <class Src, typename TW>
inline void launch_up_rows(const Src& src, int64_t T, int H, const void* w_uv, void* out,
                           int out_dtype, hipStream_t stream) {
  if (out_dtype == LCA_BF16) launch_up_rows_typed<Src, TW, bf16_t>(src, T, H, w_uv, out, stream);
  else launch_up_rows_typed<Src, TW, float>(src, T, H, w_uv, out, stream);
}

}  // namespace lca
