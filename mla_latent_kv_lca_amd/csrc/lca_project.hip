// The projection step in front of the latent attention, gfx950.
//
// MLA stores one down-projected latent per token and keeps the rotary part
// of the key as a separate, decoupled 64-wide vector ("新一代开源大模型架构演进
// 与注意力机制深度对比解析", 三.1, where RoPE also needs its own handling; the
// LCT page's 研究背景与动机 / 核心矛盾 names the two parts C^KV and K^R). For a
// hidden state x_t at position p_t this step produces
//   the cache row   [c_t ; RoPE(k_t, p_t)],  c_t = W_DKV x_t,  k_t = W_KR x_t,
//   per head h      [q^nope ; q^rope] = W_Q[h] x_t,
//   the absorbed query [W_UK[h] q^nope ; RoPE(q^rope, p_t)]
// and writes the cache row straight into the caller's cache (the append).
// RoPE rotates dimension pairs (i, i + 32) by p theta_i, theta_i =
// base^(-i/32).
//
// Two MFMA GEMMs of the same shape class, out[t][n] = sum_k A[t][k] B[n][k]
// with both operands k-contiguous:
//   1. x [T, d] against the projection weights [576 + 192 H, d]. Output
//      columns are taken in 128-wide blocks: 4 blocks of c, H blocks of
//      per-head q^nope, then the rotary segments (k^R, then q^rope of each
//      head) two 64-wide segments per block. Since a weight row is the whole
//      weight vector of one output column, any grouping of columns into
//      blocks costs nothing, and it puts both halves of a rotary pair in
//      the same lane of the same wave: the rotation happens in registers.
//   2. q^nope [T, H, 128] (bf16, from the workspace) against W_UK[h]
//      [512, 128], one head per grid z.
// A workgroup of 4 wavefronts computes a 128 x 128 output tile; each wave a
// 64 x 64 quarter with four 32x32x16 MFMA chains. Both operands stream
// HBM -> LDS with direct loads in 32-deep k slices through a 4-slice ring
// (three slices in flight while one is consumed).
#include "lca_stream.h"
#include "lca_internal.h"

namespace lca {

constexpr int PJ_BM = 128;                       // tokens per tile
constexpr int PJ_BN = 128;                       // output columns per tile
constexpr int PJ_BK = 32;                        // k per LDS slice
constexpr int PJ_NBUF = 4;                       // ring depth (slices)
constexpr int PJ_SLOTS = PJ_BM * PJ_BK / 8;      // 16-byte slots per operand slice (512)
constexpr int PJ_SLICE = 2 * PJ_SLOTS * 8;       // bf16 per slice, both operands (16 KB)
constexpr int PJ_DMA = PJ_SLOTS / 64 / 4;        // direct loads per operand, wave and slice (2)
static_assert(PJ_BM == PJ_BN, "operand slices share one slot layout");

// Slot layout of an operand slice: row r (a token, or an output column) has
// its 4 chunks of 8 k values at slots 4 r + (c ^ pj_swz(r)). The 16 rows read
// by 16 consecutive lanes then cover all 64 banks once.
__device__ __forceinline__ int pj_swz(int r) { return (r >> 2) & 3; }

// Per-lane base pointers of the direct loads: slot P = 64 (w + 4 i) + lane of
// an operand slice holds row 16 (w + 4 i) + lane / 4, chunk (lane & 3) ^
// (lane >> 4) & 3 (that row's pj_swz).
__device__ __forceinline__ int pj_dma_row(int w, int i, int lane) { return 16 * (w + 4 * i) + (lane >> 2); }
__device__ __forceinline__ int pj_dma_chunk(int lane) { return (lane & 3) ^ ((lane >> 4) & 3); }

__device__ __forceinline__ void pj_wait(int newer) {  // 4 direct loads per slice and wave
  if (newer >= 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (newer == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// acc[mt][nt][i] = sum_k A[row 64 wm + 32 mt + 8 (i / 4) + 4 (lane / 32) + i % 4][k]
//                      * B[row 64 wn + 32 nt + lane % 32][k],   w = 2 wm + wn.
__device__ __forceinline__ void pj_mainloop(bf16_t* ring, const bf16_t* const (&ap)[PJ_DMA],
                                            const bf16_t* const (&bp)[PJ_DMA], int K, int w, int lane,
                                            f32x16_t (&acc)[2][2]) {
  const int wm = w >> 1, wn = w & 1;
  const int nk = K / PJ_BK;
  const uint32_t ring0 = lds_off(ring);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

  auto issue = [&](int s) {
    const uint32_t buf = ring0 + (uint32_t)((s % PJ_NBUF) * PJ_SLICE * 2);
    const int k0 = s * PJ_BK;
#pragma unroll
    for (int i = 0; i < PJ_DMA; ++i) dma16(ap[i] + k0, buf + 1024u * (uint32_t)(w + 4 * i));
#pragma unroll
    for (int i = 0; i < PJ_DMA; ++i) dma16(bp[i] + k0, buf + PJ_SLOTS * 16u + 1024u * (uint32_t)(w + 4 * i));
  };
  for (int s = 0; s < PJ_NBUF - 1 && s < nk; ++s) issue(s);

  // fragment offsets (bf16 elements within an operand slice): row 32 x + lane % 32,
  // chunk 2 kk + lane / 32, whose swizzle is (lane >> 2) & 3
  const int r32 = lane & 31, sw = (lane >> 2) & 3, hk = lane >> 5;
  int fo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) fo[kk] = 8 * (4 * r32 + ((2 * kk + hk) ^ sw));

  for (int s = 0; s < nk; ++s) {
    pj_wait(min(nk - 1 - s, PJ_NBUF - 2));
    barrier();  // slice s landed for every wave; slice s - 1 is consumed by every wave
    if (s + PJ_NBUF - 1 < nk) issue(s + PJ_NBUF - 1);
    const bf16_t* A = ring + (s % PJ_NBUF) * PJ_SLICE;
    const bf16_t* B = A + PJ_SLOTS * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 a[2], b[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        a[mt] = *reinterpret_cast<const uint4*>(A + 8 * 4 * (64 * wm + 32 * mt) + fo[kk]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        b[nt] = *reinterpret_cast<const uint4*>(B + 8 * 4 * (64 * wn + 32 * nt) + fo[kk]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32x32x16(a[mt], b[nt], acc[mt][nt]);
    }
  }
}

struct ProjArgs {
  const bf16_t* x;       // [T, d] hidden states, row stride x_stride
  int64_t x_stride;
  int64_t T;
  int d;                 // model width, a multiple of PJ_BK
  int H;
  const int32_t* pos;    // [T] positions
  double log2_base;      // log2 of the RoPE base
  const bf16_t* w;       // [576 + 192 H, d] projection weights (one row per output column)
  bf16_t* rows;          // cache rows, token t's row at rows + dst_row[t] * row_stride
  int64_t row_stride;
  const int64_t* dst_row;
  void* q;               // absorbed queries, token t head h at q + t * q_stride + 576 h
  int64_t q_stride;
  bf16_t* qn;            // [T, H, 128] q^nope for the absorption
};

// Weight row of local column j (0..127) of column block nb.
__device__ __forceinline__ int64_t proj_wrow(int nb, int j, int H) {
  if (nb < 4) return 128 * nb + j;                               // c
  if (nb < 4 + H) return D_ROW + 192 * (nb - 4) + j;             // q^nope of head nb - 4
  int s = 2 * (nb - 4 - H) + (j >> 6);                           // rotary segment
  if (s > H) s = H;  // the unused half of the last block: any valid row
  const int dd = j & 63;
  return s == 0 ? D_C + dd : D_ROW + 192 * (s - 1) + 128 + dd;
}

// cos and sin of p theta_d, theta_d = 2^(-d log2(base) / 32). The angle is
// formed and reduced to [-pi, pi] in double (positions reach millions of
// radians), then evaluated in float.
__device__ __forceinline__ void rope_cs(int32_t p, double theta, float& c, float& s) {
  const double a = (double)p * theta;
  const double k = rint(a * 0.15915494309189535);        // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, a);              // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);                // 2 pi, low part
  sincosf((float)r, &s, &c);
}

template <typename TQ>
__global__ __launch_bounds__(256, 2) void proj_kernel(ProjArgs pa) {
  __shared__ __align__(16) bf16_t ring[PJ_NBUF * PJ_SLICE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = blockIdx.y;
  const int64_t tok0 = (int64_t)blockIdx.x * PJ_BM;

  const bf16_t* ap[PJ_DMA];
  const bf16_t* bp[PJ_DMA];
  const int ch = pj_dma_chunk(lane);
#pragma unroll
  for (int i = 0; i < PJ_DMA; ++i) {
    const int r = pj_dma_row(w, i, lane);
    const int64_t t = min(tok0 + r, pa.T - 1);  // rows past T load a valid row; never stored
    ap[i] = pa.x + t * pa.x_stride + 8 * ch;
    bp[i] = pa.w + proj_wrow(nb, r, pa.H) * pa.d + 8 * ch;
  }
  f32x16_t acc[2][2];
  pj_mainloop(ring, ap, bp, pa.d, w, lane, acc);

  const int wm = w >> 1, wn = w & 1, r32 = lane & 31, hk = lane >> 5;
  const int H = pa.H;
  if (nb < 4 + H) {  // c -> cache rows, or q^nope -> workspace (bf16)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t t = tok0 + 64 * wm + 32 * mt + 8 * (i >> 2) + 4 * hk + (i & 3);
        if (t >= pa.T) continue;
        bf16_t* dst;
        if (nb < 4) {
          const int64_t dr = pa.dst_row[t];
          if (dr < 0) continue;
          dst = pa.rows + dr * pa.row_stride + 128 * nb;
        } else {
          dst = pa.qn + (t * H + (nb - 4)) * D_V;
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) dst[64 * wn + 32 * nt + r32] = (bf16_t)f2bf(acc[mt][nt][i]);
      }
    return;
  }
  const int s = 2 * (nb - 4 - H) + wn;  // this wave's rotary segment: 0 = k^R, 1 + h = q^rope of head h
  if (s > H) return;
  const double theta = exp2(-(double)r32 * (1.0 / 32.0) * pa.log2_base);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t t = tok0 + 64 * wm + 32 * mt + 8 * (i >> 2) + 4 * hk + (i & 3);
      if (t >= pa.T) continue;
      float cs, sn;
      rope_cs(pa.pos[t], theta, cs, sn);
      const float x1 = acc[mt][0][i], x2 = acc[mt][1][i];
      const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
      if (s == 0) {
        const int64_t dr = pa.dst_row[t];
        if (dr < 0) continue;
        bf16_t* dst = pa.rows + dr * pa.row_stride + D_C;
        dst[r32] = (bf16_t)f2bf(y1);
        dst[32 + r32] = (bf16_t)f2bf(y2);
      } else {
        TQ* dst = reinterpret_cast<TQ*>(pa.q) + t * pa.q_stride + (int64_t)(s - 1) * D_ROW + D_C;
        dst[r32] = from_f32<TQ>(y1);
        dst[32 + r32] = from_f32<TQ>(y2);
      }
    }
}

// q_abs[t, h, 128 jb + j] = sum_k qn[t, h, k] W_UK[h][128 jb + j][k]
template <typename TQ>
__global__ __launch_bounds__(256, 2) void absorb_kernel(const bf16_t* __restrict__ qn, int64_t T, int H,
                                                        const bf16_t* __restrict__ wuk, void* q,
                                                        int64_t q_stride) {
  __shared__ __align__(16) bf16_t ring[PJ_NBUF * PJ_SLICE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jb = blockIdx.y, h = blockIdx.z;
  const int64_t tok0 = (int64_t)blockIdx.x * PJ_BM;

  const bf16_t* ap[PJ_DMA];
  const bf16_t* bp[PJ_DMA];
  const int ch = pj_dma_chunk(lane);
#pragma unroll
  for (int i = 0; i < PJ_DMA; ++i) {
    const int r = pj_dma_row(w, i, lane);
    const int64_t t = min(tok0 + r, T - 1);
    ap[i] = qn + (t * H + h) * D_V + 8 * ch;
    bp[i] = wuk + ((int64_t)h * D_C + PJ_BN * jb + r) * D_V + 8 * ch;
  }
  f32x16_t acc[2][2];
  pj_mainloop(ring, ap, bp, D_V, w, lane, acc);

  const int wm = w >> 1, wn = w & 1, r32 = lane & 31, hk = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t t = tok0 + 64 * wm + 32 * mt + 8 * (i >> 2) + 4 * hk + (i & 3);
      if (t >= T) continue;
      TQ* dst = reinterpret_cast<TQ*>(q) + t * q_stride + (int64_t)h * D_ROW + PJ_BN * jb + 64 * wn + r32;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) dst[32 * nt] = from_f32<TQ>(acc[mt][nt][i]);
    }
}

hipError_t launch_project(const void* x, int64_t x_stride, int64_t T, int d, const int32_t* pos,
                          double rope_base, const void* w_proj, const void* w_uk, int H, void* rows,
                          int64_t row_stride, const int64_t* dst_row, void* q, int q_dtype,
                          int64_t q_stride, void* qn, hipStream_t stream) {
  ProjArgs pa{(const bf16_t*)x, x_stride, T, d, H, pos, log2(rope_base), (const bf16_t*)w_proj,
              (bf16_t*)rows, row_stride, dst_row, q, q_stride, (bf16_t*)qn};
  const unsigned tiles = (unsigned)((T + PJ_BM - 1) / PJ_BM);
  const dim3 g1(tiles, (unsigned)(4 + H + (H + 2) / 2));
  const dim3 g2(tiles, D_C / PJ_BN, (unsigned)H);
  if (q_dtype == LCA_BF16) {
    hipLaunchKernelGGL(proj_kernel<bf16_t>, g1, dim3(256), 0, stream, pa);
    hipLaunchKernelGGL(absorb_kernel<bf16_t>, g2, dim3(256), 0, stream, (const bf16_t*)qn, T, H,
                       (const bf16_t*)w_uk, q, q_stride);
  } else {
    hipLaunchKernelGGL(proj_kernel<float>, g1, dim3(256), 0, stream, pa);
    hipLaunchKernelGGL(absorb_kernel<float>, g2, dim3(256), 0, stream, (const bf16_t*)qn, T, H,
                       (const bf16_t*)w_uk, q, q_stride);
  }
  return hipGetLastError();
}

}  // namespace lca
