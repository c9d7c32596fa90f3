// LCA condensation kernels for gfx950.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// 关键设计 1 (summary query = mean of the most recent g queries, per-token
// importance, softmax weights, weighted pooling of c_KV) and 关键设计 2 (the
// group's k_R is the k_R of its most important token).
//
// Two kernels:
//  qbar_kernel      one workgroup per summary query: mean over g query tokens
//                   and H heads of 576-wide absorbed queries -> fp32 workspace.
//  condense_kernel  one wavefront per group. Lane l owns latent columns
//                   [8l, 8l+8) and RoPE column l of all g rows, so each row
//                   load is one fully coalesced 1 KB (c_KV) + 128 B (k_R)
//                   wave access and every row's score is formed by the same
//                   sequence of operations (identical rows give bitwise equal
//                   scores). The g partial dot products are reduced across
//                   the 64 lanes with a halving butterfly (g/2 + g/4 + ...
//                   shuffles instead of 6 g), the g-way softmax / argmax uses
//                   shuffles, and the pooled row is accumulated in fp32.
// The work is HBM streaming (about 2 flop per byte): no matrix cores.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

// ---------------------------------------------------------------- K0 -------
constexpr int QBAR_PH = 14;                  // row phases
constexpr int QBAR_THREADS = 72 * QBAR_PH;   // 72 column chunks of 8 x 14 row phases

// One workgroup per summary query: thread (chunk c, phase p) sums rows
// p, p + 14, ... of the g*H query rows, eight loads in flight at a time; the
// 14 phase partials are then added in phase order.
template <typename TQ>
__global__ __launch_bounds__(QBAR_THREADS) void qbar_kernel(
    const TQ* __restrict__ q, int64_t q_seq, int64_t q_tok, int H, int g, int64_t row0,
    int64_t step, int n_q, float* __restrict__ qbar) {
  const int jq = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, ch = t % 72, ph = t / 72;
  const TQ* base = q + (int64_t)b * q_seq + (row0 + (int64_t)jq * step) * q_tok + ch * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int rows = g * H;
  for (int r0 = ph; r0 < rows; r0 += 8 * QBAR_PH) {
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * QBAR_PH;
      if (r < rows) {
        const int tok = r / H, h = r - tok * H;
        load8_f32(base + (int64_t)tok * q_tok + h * D_ROW, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[u][i];
  }
  __shared__ float sh[QBAR_PH][D_ROW];
#pragma unroll
  for (int i = 0; i < 8; ++i) sh[ph][ch * 8 + i] = acc[i];
  __syncthreads();
  const float inv = 1.0f / (float)rows;
  for (int c = t; c < D_ROW; c += QBAR_THREADS) {
    float s = sh[0][c];
    for (int p = 1; p < QBAR_PH; ++p) s += sh[p][c];
    qbar[((int64_t)b * n_q + jq) * D_ROW + c] = s * inv;
  }
}

// ---------------------------------------------------------------- K1 -------
// Reduce v[0..G) over all 64 lanes; afterwards every lane holds the total of
// row (lane >> (6 - LG)).
template <int LG>
__device__ __forceinline__ float reduce_rows(float (&v)[1 << LG], int lane) {
  constexpr int G = 1 << LG;
#pragma unroll
  for (int st = 0; st < LG; ++st) {
    const int mask = 32 >> st;
    const int half = G >> (st + 1);
    const bool upper = (lane & mask) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? v[i] : v[i + half];
      const float keep = upper ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, mask);
    }
  }
  float x = v[0];
#pragma unroll
  for (int mask = 32 >> LG; mask >= 1; mask >>= 1) x += __shfl_xor(x, mask);
  return x;
}

template <typename TC> struct RowChunk;  // 8 latent elements of one row held by a lane
template <> struct RowChunk<bf16_t> {
  uint4 v;
  __device__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ float get(int i) const {
    const uint32_t w = u4_get(v, i >> 1);
    return (i & 1) ? bf_hi(w) : bf_lo(w);
  }
};
template <> struct RowChunk<float> {
  float v[8];
  __device__ void load(const float* p) { load8_f32(p, v); }
  __device__ float get(int i) const { return v[i]; }
};

template <typename TC, typename TR, int LG>
__global__ __launch_bounds__(256) void condense_kernel(
    const TC* __restrict__ c, const TC* __restrict__ kr, int64_t c_seq, int64_t c_tok,
    int64_t kr_seq, int64_t kr_tok, const float* __restrict__ qbar, int per_group_q,
    int64_t n_q, int64_t group_begin, int64_t n_groups, float sm_scale, TR* __restrict__ rc,
    TR* __restrict__ rk, int64_t rc_seq, int64_t rc_tok, int64_t rk_seq, int64_t rk_tok,
    int32_t* __restrict__ anchor, int64_t anchor_seq, float* __restrict__ alpha,
    int64_t alpha_seq) {
  constexpr int G = 1 << LG;
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_groups) return;  // wave-uniform
  const int b = blockIdx.y;
  const int64_t j = group_begin + n;

  const float* qb = qbar + ((int64_t)b * n_q + (per_group_q ? n : 0)) * D_ROW;
  float qc[8];
  load8_f32(qb + 8 * lane, qc);
  const float qr = qb[D_C + lane];

  const TC* cg = c + (int64_t)b * c_seq + j * G * c_tok + 8 * lane;
  const TC* kg = kr + (int64_t)b * kr_seq + j * G * kr_tok + lane;
  RowChunk<TC> rows[G];
  TC krv[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    rows[r].load(cg + r * c_tok);
    krv[r] = kg[r * kr_tok];
  }

  // partial scores of this lane's columns, same operation order for every row
  float s[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    float a = rows[r].get(0) * qc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) a = fmaf(rows[r].get(i), qc[i], a);
    s[r] = fmaf(to_f32(krv[r]), qr, a);
  }
  const float score = reduce_rows<LG>(s, lane);
  const int my_row = lane >> (6 - LG);

  // group max and first argmax over rows (rows sit in the top LG lane bits)
  float mx = score;
  int arg = my_row;
#pragma unroll
  for (int st = 0; st < LG; ++st) {
    const int mask = 32 >> st;
    const float om = __shfl_xor(mx, mask);
    const int oa = __shfl_xor(arg, mask);
    if (om > mx || (om == mx && oa < arg)) { mx = om; arg = oa; }
  }
  const float e = __expf(sm_scale * (score - mx));
  float tot = e;
#pragma unroll
  for (int st = 0; st < LG; ++st) tot += __shfl_xor(tot, 32 >> st);
  const float a_mine = e / tot;

  // pooled latent: sum_r alpha_r c_r in row order
  float acc[8];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const float ar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a_mine), r << (6 - LG)));
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (r == 0) ? ar * rows[r].get(i) : fmaf(ar, rows[r].get(i), acc[i]);
  }
  store8(rc + (int64_t)b * rc_seq + j * rc_tok + 8 * lane, acc);

  // anchor row's k_R (arg is uniform across the wave)
  TC ksel = krv[0];
#pragma unroll
  for (int r = 1; r < G; ++r) ksel = (r == arg) ? krv[r] : ksel;
  rk[(int64_t)b * rk_seq + j * rk_tok + lane] = from_f32<TR>(to_f32(ksel));
  if (lane == 0) anchor[(int64_t)b * anchor_seq + j] = (int32_t)(j * G + arg);
  if (alpha != nullptr && (lane & ((64 >> LG) - 1)) == 0)
    alpha[(int64_t)b * alpha_seq + j * G + my_row] = a_mine;
}

template <typename TC, typename TR, int LG>
static void launch_k1(dim3 grid, hipStream_t st, const lca_latent_t& cache, const float* qbar,
                      int per_group_q, int64_t n_q, int64_t gb, int64_t ng, float sm,
                      const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq,
                      float* alpha, int64_t alpha_seq) {
  hipLaunchKernelGGL((condense_kernel<TC, TR, LG>), grid, dim3(256), 0, st,
                     (const TC*)cache.c, (const TC*)cache.kr, cache.c_seq_stride,
                     cache.c_tok_stride, cache.kr_seq_stride, cache.kr_tok_stride, qbar,
                     per_group_q, n_q, gb, ng, sm, (TR*)reps.c, (TR*)reps.kr, reps.c_seq_stride,
                     reps.c_tok_stride, reps.kr_seq_stride, reps.kr_tok_stride, anchor,
                     anchor_seq, alpha, alpha_seq);
}

template <typename TC, typename TR>
static void dispatch_g(int lg, dim3 grid, hipStream_t st, const lca_latent_t& cache,
                       const float* qbar, int pg, int64_t n_q, int64_t gb, int64_t ng, float sm,
                       const lca_latent_t& reps, int32_t* anchor, int64_t as, float* alpha,
                       int64_t als) {
  switch (lg) {
    case 0: launch_k1<TC, TR, 0>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    case 1: launch_k1<TC, TR, 1>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    case 2: launch_k1<TC, TR, 2>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    case 3: launch_k1<TC, TR, 3>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    case 4: launch_k1<TC, TR, 4>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    default: launch_k1<TC, TR, 5>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
  }
}

hipError_t launch_condense(const lca_latent_t& cache, int B, int g, int64_t group_begin,
                           int64_t n_groups, const void* q, int q_dtype, int64_t q_seq_stride,
                           int64_t q_tok_stride, int H, int64_t q_row0, int64_t q_row_step,
                           float sm_scale, const lca_latent_t& reps, int32_t* anchor,
                           int64_t anchor_seq, float* alpha, int64_t alpha_seq, float* qbar_ws,
                           hipStream_t stream) {
  const int per_group_q = q_row_step != 0;
  const int64_t n_q = per_group_q ? n_groups : 1;
  dim3 g0((unsigned)n_q, (unsigned)B);
  if (q_dtype == LCA_BF16)
    hipLaunchKernelGGL(qbar_kernel<bf16_t>, g0, dim3(QBAR_THREADS), 0, stream, (const bf16_t*)q,
                       q_seq_stride, q_tok_stride, H, g, q_row0, q_row_step, (int)n_q, qbar_ws);
  else
    hipLaunchKernelGGL(qbar_kernel<float>, g0, dim3(QBAR_THREADS), 0, stream, (const float*)q,
                       q_seq_stride, q_tok_stride, H, g, q_row0, q_row_step, (int)n_q, qbar_ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  int lg = 0;
  while ((1 << lg) < g) ++lg;
  dim3 g1((unsigned)((n_groups + 3) / 4), (unsigned)B);
  const bool cb = cache.dtype == LCA_BF16, rb = reps.dtype == LCA_BF16;
  if (cb && rb)
    dispatch_g<bf16_t, bf16_t>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq);
  else if (cb)
    dispatch_g<bf16_t, float>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq);
  else if (rb)
    dispatch_g<float, bf16_t>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq);
  else
    dispatch_g<float, float>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq);
  return hipGetLastError();
}

}  // namespace lca
