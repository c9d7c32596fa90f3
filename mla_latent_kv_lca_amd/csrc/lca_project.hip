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
//   1. x [T, d] against the projection weights [576 + 192 H, d], with the
//      rotation and the scatter of the cache rows in the epilogue. Since a
//      weight row is the whole weight vector of one output column, any
//      grouping of output columns into tiles costs nothing: the tiles put
//      both halves of a rotary pair in the same lane, so the rotation
//      happens in registers.
//   2. q^nope [T, H, 128] (bf16, through the workspace) against W_UK[h]
//      [512, 128].
// By token count:
//   - up to 64 tokens (decode): proj_rows_kernel / absorb_rows_kernel,
//     16 output columns per workgroup over the whole model width, every
//     load of a wave in flight at once (HBM-bound on the weights);
//   - more: proj_kernel (fewer than about 4,096 tokens: 128 x 128 tiles, 4
//     wavefronts of 64 x 64, four 32x32x16 chains) or proj_big_kernel (256 x
//     256 tiles, 8 wavefronts of 128 x 64), which stream both operands
//     HBM -> LDS by direct loads in 32-deep k slices through a 4-slice ring
//     (three slices in flight while one is consumed); then
//     absorb_stream_kernel, persistent per head with W_UK[h] in registers.
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
    uint4 a[2][2], b[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        a[kk][mt] = *reinterpret_cast<const uint4*>(A + 8 * 4 * (64 * wm + 32 * mt) + fo[kk]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        b[kk][nt] = *reinterpret_cast<const uint4*>(B + 8 * 4 * (64 * wn + 32 * nt) + fo[kk]);
    }
    __builtin_amdgcn_sched_barrier(0);  // all 8 reads in flight before the first product
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32x32x16(a[kk][mt], b[kk][nt], acc[mt][nt]);
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

// Rotation frequency of pair i in turns per position: base^(-i/32) / (2 pi).
__device__ __forceinline__ double rope_turns(int i, double log2_base) {
  return exp2(-(double)i * (1.0 / 32.0) * log2_base) * 0.15915494309189535;
}
// cos and sin of the angle p theta_i. The angle in turns, p * turns, is formed
// and reduced to [-1/2, 1/2] in double (positions reach millions of
// radians), then the hardware sine and cosine, whose inputs are in turns,
// evaluate it.
__device__ __forceinline__ void rope_cs(int32_t p, double turns, float& c, float& s) {
  const double a = (double)p * turns;
  const float r = (float)(a - rint(a));
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
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
  const double turns = rope_turns(r32, pa.log2_base);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t t = tok0 + 64 * wm + 32 * mt + 8 * (i >> 2) + 4 * hk + (i & 3);
      if (t >= pa.T) continue;
      float cs, sn;
      rope_cs(pa.pos[t], turns, cs, sn);
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

// ---- many tokens: 256 x 256 output tiles. Eight wavefronts (two per SIMD,
// so one wave's waits overlap the other's products) of 128 tokens x 64
// columns: eight 32x32x16 chains each (128 accumulator registers). Both operands
// stream HBM -> LDS by direct loads in 32-deep k slices through a 4-slice
// ring (128 KB), three slices in flight; per slice a wave issues its 12
// fragment reads for both k steps before its 16 products. Output columns in
// 256-wide blocks: 2 of c, one per two heads of q^nope, then the rotary
// segments four per block, one per wave column (so again both halves of a
// pair meet in one lane).
constexpr int PB_BM = 256;                       // tokens per tile
static_assert(PB_BM == 256, "a tile is 256 tokens x 256 output columns");
constexpr int PB_WAVES = 8;
constexpr int PB_SLOTS = PB_BM * PJ_BK / 8;      // 16-byte slots per operand slice (1024)
constexpr int PB_SLICE = 2 * PB_SLOTS * 8;       // bf16 per slice, both operands (32 KB)
constexpr int PB_DMA = PB_SLOTS / 64 / PB_WAVES; // direct loads per operand, wave and slice (2)

// acc[mt][nt][i] = sum_k A[row 128 wm + 32 mt + 8 (i / 4) + 4 (lane / 32) + i % 4][k]
//                      * B[row 64 wn + 32 nt + lane % 32][k],   w = 4 wm + wn.
__device__ __forceinline__ void pb_mainloop(bf16_t* ring, const bf16_t* const (&ap)[PB_DMA],
                                            const bf16_t* const (&bp)[PB_DMA], int K, int w, int lane,
                                            f32x16_t (&acc)[4][2]) {
  const int wm = w >> 2, wn = w & 3;
  const int nk = K / PJ_BK;
  const uint32_t ring0 = lds_off(ring);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

  auto issue = [&](int s) {
    const uint32_t buf = ring0 + (uint32_t)((s % PJ_NBUF) * PB_SLICE * 2);
    const int k0 = s * PJ_BK;
#pragma unroll
    for (int i = 0; i < PB_DMA; ++i) dma16(ap[i] + k0, buf + 1024u * (uint32_t)(w + PB_WAVES * i));
#pragma unroll
    for (int i = 0; i < PB_DMA; ++i)
      dma16(bp[i] + k0, buf + PB_SLOTS * 16u + 1024u * (uint32_t)(w + PB_WAVES * i));
  };
  for (int s = 0; s < PJ_NBUF - 1 && s < nk; ++s) issue(s);

  const int r32 = lane & 31, sw = (lane >> 2) & 3, hk = lane >> 5;
  int fo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) fo[kk] = 8 * (4 * r32 + ((2 * kk + hk) ^ sw));

  for (int s = 0; s < nk; ++s) {
    pj_wait(min(nk - 1 - s, PJ_NBUF - 2));  // 4 direct loads per slice and wave, as in the 128 tiles
    barrier();  // slice s landed for every wave; slice s - 1 is consumed by every wave
    if (s + PJ_NBUF - 1 < nk) issue(s + PJ_NBUF - 1);
    const bf16_t* A = ring + (s % PJ_NBUF) * PB_SLICE + 8 * 4 * 128 * wm;
    const bf16_t* B = ring + (s % PJ_NBUF) * PB_SLICE + PB_SLOTS * 8 + 8 * 4 * 64 * wn;
    uint4 a[2][4], b[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a[kk][mt] = *reinterpret_cast<const uint4*>(A + 8 * 4 * 32 * mt + fo[kk]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) b[kk][nt] = *reinterpret_cast<const uint4*>(B + 8 * 4 * 32 * nt + fo[kk]);
    }
    // all 12 reads in flight before the first product: the compiler would
    // otherwise interleave them one by one and wait on each
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32x32x16(a[kk][mt], b[kk][nt], acc[mt][nt]);
  }
}

// Weight row of local column j (0..255) of a 256-wide column block.
__device__ __forceinline__ int64_t big_wrow(int nb, int j, int H) {
  if (nb < 2) return 256 * nb + j;                                  // c
  const int nh = (H + 1) / 2;
  if (nb < 2 + nh) {                                                // q^nope of heads 2 (nb - 2) + j / 128
    const int h = min(2 * (nb - 2) + (j >> 7), H - 1);             // the unused half of an odd H: a valid row
    return D_ROW + 192 * h + (j & 127);
  }
  const int s = min(4 * (nb - 2 - nh) + (j >> 6), H);              // rotary segment
  const int dd = j & 63;
  return s == 0 ? D_C + dd : D_ROW + 192 * (s - 1) + 128 + dd;
}

// Tile order of proj_big_kernel. Workgroups are dealt to the 8 XCDs round
// robin (workgroup b runs on XCD b % 8), so XCD k takes the contiguous run
// [k c, k c + c) of a tile order that walks groups of PB_GX token tiles
// column block by column block: each XCD's L2 then serves about PB_GX token
// tiles and a share of the weight columns, instead of two token tiles and
// every weight column (x fastest). Measured at 4,096 tokens, d = 2,048,
// H = 16: L2 misses drop from 137 to 98 MB per call while the call time stays
// the same (the loop is bound by its own instruction stream, not by these
// re-reads).
constexpr int PB_GX = 4;
__host__ __device__ inline int pb_columns(int H) { return 2 + (H + 1) / 2 + (H + 4) / 4; }
__device__ __forceinline__ bool pb_tile_of(int b, int nx, int ny, int& x, int& y) {
  const int n = nx * ny, c = (n + 7) / 8;
  const int L = (b & 7) * c + (b >> 3);
  if (L >= n) return false;
  const int gsize = PB_GX * ny, g = L / gsize, r = L - g * gsize;
  const int x0 = g * PB_GX, gw = min(PB_GX, nx - x0);
  y = r / gw;
  x = x0 + r - y * gw;
  return true;
}

template <typename TQ>
__global__ __launch_bounds__(64 * PB_WAVES, 2) void proj_big_kernel(ProjArgs pa) {
  __shared__ __align__(16) bf16_t ring[PJ_NBUF * PB_SLICE];
  // the tile's destination rows and positions: loaded before the main loop,
  // shared through LDS after it (in the epilogue each would otherwise be a
  // global load ordered after the previous token's stores)
  __shared__ int64_t tile_dst[PB_BM];
  __shared__ int32_t tile_pos[PB_BM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = pa.H;
  int bx, nb;
  if (!pb_tile_of((int)blockIdx.x, (int)((pa.T + PB_BM - 1) / PB_BM), pb_columns(H), bx, nb)) return;
  const int64_t tok0 = (int64_t)bx * PB_BM;
  int64_t my_dst = 0;
  int32_t my_pos = 0;
  if (tid < PB_BM) {
    const int64_t t = min(tok0 + tid, pa.T - 1);
    my_dst = pa.dst_row[t];
    my_pos = pa.pos[t];
  }

  const bf16_t* ap[PB_DMA];
  const bf16_t* bp[PB_DMA];
  const int ch = pj_dma_chunk(lane);
#pragma unroll
  for (int i = 0; i < PB_DMA; ++i) {
    const int r = 16 * (w + PB_WAVES * i) + (lane >> 2);  // slot 64 (w + 8 i) + lane
    const int64_t t = min(tok0 + r, pa.T - 1);            // rows past T load a valid row; never stored
    ap[i] = pa.x + t * pa.x_stride + 8 * ch;
    bp[i] = pa.w + big_wrow(nb, r, H) * pa.d + 8 * ch;
  }
  f32x16_t acc[4][2];
  pb_mainloop(ring, ap, bp, pa.d, w, lane, acc);
  if (tid < PB_BM) {
    tile_dst[tid] = my_dst;
    tile_pos[tid] = my_pos;
  }
  __syncthreads();

  const int wm = w >> 2, wn = w & 3, r32 = lane & 31, hk = lane >> 5;
  const int nh = (H + 1) / 2;
  if (nb < 2 + nh) {  // c -> cache rows, or q^nope -> workspace (bf16)
    const int h = 2 * (nb - 2) + (wn >> 1);
    if (nb >= 2 && h >= H) return;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tl = 128 * wm + 32 * mt + 8 * (i >> 2) + 4 * hk + (i & 3);
        const int64_t t = tok0 + tl;
        if (t >= pa.T) continue;
        bf16_t* dst;
        if (nb < 2) {
          const int64_t dr = tile_dst[tl];
          if (dr < 0) continue;
          dst = pa.rows + dr * pa.row_stride + 256 * nb + 64 * wn;
        } else {
          dst = pa.qn + (t * H + h) * D_V + 64 * (wn & 1);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) dst[32 * nt + r32] = (bf16_t)f2bf(acc[mt][nt][i]);
      }
    return;
  }
  const int s = 4 * (nb - 2 - nh) + wn;  // this wave's rotary segment: 0 = k^R, 1 + h = q^rope of head h
  if (s > H) return;
  const double turns = rope_turns(r32, pa.log2_base);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tl = 128 * wm + 32 * mt + 8 * (i >> 2) + 4 * hk + (i & 3);
      const int64_t t = tok0 + tl;
      if (t >= pa.T) continue;
      float cs, sn;
      rope_cs(tile_pos[tl], turns, cs, sn);
      const float x1 = acc[mt][0][i], x2 = acc[mt][1][i];
      const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
      if (s == 0) {
        const int64_t dr = tile_dst[tl];
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

// ---- few tokens (decode): the weights stream once, spread over many
// workgroups. A workgroup computes 16 output columns for up to 32 tokens over
// the whole model width. The width is cut into 256-wide k chunks dealt to the
// 8 wavefronts round-robin; per chunk a wave issues all of its loads at once
// (one memory round trip): the 32 x 256 hidden-state block goes to the wave's
// own LDS region by direct loads that read whole 512-byte row pieces, and the
// 16 weight rows go straight into MFMA operand registers. The 8 partial tiles
// are added in wave order through LDS and the epilogue runs on the sums.
// Columns are grouped 16 at a time: 32 groups of c, 8 per head of q^nope,
// then 4 per rotary segment holding the dimension pairs (8 u + i, 32 + 8 u +
// i), i < 8.
constexpr int PR_TOK = 32;    // tokens per workgroup
constexpr int PR_COLS = 16;   // output columns per workgroup
constexpr int PR_WAVES = 8;   // wavefronts per workgroup
constexpr int PR_KC = 256;    // k per chunk
constexpr int PR_MAX_T = 64;  // token counts up to this take this path
constexpr int PR_XSLOTS = PR_TOK * PR_KC / 8;  // 16-byte slots of one wave's hidden-state block (1024)

__device__ __forceinline__ int64_t rows_wrow(int cg, int j, int H) {
  if (cg < D_C / PR_COLS) return PR_COLS * cg + j;                        // c
  cg -= D_C / PR_COLS;
  if (cg < 8 * H) return D_ROW + 192 * (cg >> 3) + PR_COLS * (cg & 7) + j;  // q^nope
  cg -= 8 * H;
  const int s = cg >> 2, u = cg & 3;                                      // rotary segment, quarter
  const int dd = j < 8 ? 8 * u + j : 32 + 8 * u + (j - 8);
  return s == 0 ? D_C + dd : D_ROW + 192 * (s - 1) + 128 + dd;
}

__global__ __launch_bounds__(64 * PR_WAVES) void proj_rows_kernel(ProjArgs pa, int q_f32) {
  // per wave: token row r of the block holds its 32 chunks with chunk c at
  // slot 32 r + (c ^ (r & 15)), so the 16 rows of an operand fragment hit 16
  // different bank groups; after the products the region holds the wave's
  // partial tile (fp32 [32][17])
  __shared__ __align__(16) bf16_t xs[PR_WAVES][PR_XSLOTS * 8];
  __shared__ float fin[PR_TOK][PR_COLS + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int cg = blockIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.y * PR_TOK;
  const int H = pa.H;

  const bf16_t* wr = pa.w + rows_wrow(cg, col, H) * pa.d + 8 * kg;
  // direct-load sources: instruction i, lane -> row 2 i + lane / 32, chunk (lane % 32) ^ (row & 15)
  const int xc = lane & 31, xrow0 = lane >> 5;
  const uint32_t xbase = lds_off(&xs[w][0]);
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  for (int ch = w; ch < pa.d / PR_KC; ch += PR_WAVES) {
    const int k0 = ch * PR_KC;
#pragma unroll
    for (int i = 0; i < PR_XSLOTS / 64; ++i) {
      const int r = 2 * i + xrow0;
      const int64_t t = min(tok0 + r, pa.T - 1);  // rows past T load a valid row; never stored
      dma16(pa.x + t * pa.x_stride + k0 + 8 * (xc ^ (r & 15)), xbase + 1024u * (uint32_t)i);
    }
    uint4 b[PR_KC / 32];
#pragma unroll
    for (int st = 0; st < PR_KC / 32; ++st) b[st] = load8_bf16(wr + k0 + 32 * st);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int st = 0; st < PR_KC / 32; ++st)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = 16 * mt + col;
        const uint4 a = *reinterpret_cast<const uint4*>(&xs[w][8 * (32 * r + ((4 * st + kg) ^ (r & 15)))]);
        acc[mt] = mfma16x16x32(a, b[st], acc[mt]);
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the block is consumed before it is reloaded
  }
  // acc[mt][r] = partial of out[token 16 mt + 4 kg + r][column col]
  float* red = reinterpret_cast<float*>(&xs[w][0]);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(16 * mt + 4 * kg + r) * (PR_COLS + 1) + col] = acc[mt][r];
  __syncthreads();
  {  // thread -> (token, column): the 8 partials in wave order
    const int tl = tid >> 4, c = tid & 15;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < PR_WAVES; ++k) v += reinterpret_cast<const float*>(&xs[k][0])[tl * (PR_COLS + 1) + c];
    fin[tl][c] = v;
  }
  __syncthreads();
  const int tl = tid >> 4, c = tid & 15;
  const int64_t t = tok0 + tl;
  if (t >= pa.T) return;
  int g = cg;
  if (g < D_C / PR_COLS) {
    const int64_t dr = pa.dst_row[t];
    if (dr >= 0) pa.rows[dr * pa.row_stride + PR_COLS * g + c] = (bf16_t)f2bf(fin[tl][c]);
    return;
  }
  g -= D_C / PR_COLS;
  if (g < 8 * H) {
    pa.qn[(t * H + (g >> 3)) * D_V + PR_COLS * (g & 7) + c] = (bf16_t)f2bf(fin[tl][c]);
    return;
  }
  g -= 8 * H;
  if (c >= 8) return;  // one thread per rotary pair
  const int s = g >> 2, i = 8 * (g & 3) + c;  // pair (i, i + 32)
  const double turns = rope_turns(i, pa.log2_base);
  float cs, sn;
  rope_cs(pa.pos[t], turns, cs, sn);
  const float x1 = fin[tl][c], x2 = fin[tl][c + 8];
  const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
  if (s == 0) {
    const int64_t dr = pa.dst_row[t];
    if (dr < 0) return;
    bf16_t* dst = pa.rows + dr * pa.row_stride + D_C;
    dst[i] = (bf16_t)f2bf(y1);
    dst[32 + i] = (bf16_t)f2bf(y2);
  } else if (q_f32) {
    float* dst = reinterpret_cast<float*>(pa.q) + t * pa.q_stride + (int64_t)(s - 1) * D_ROW + D_C;
    dst[i] = y1;
    dst[32 + i] = y2;
  } else {
    bf16_t* dst = reinterpret_cast<bf16_t*>(pa.q) + t * pa.q_stride + (int64_t)(s - 1) * D_ROW + D_C;
    dst[i] = (bf16_t)f2bf(y1);
    dst[32 + i] = (bf16_t)f2bf(y2);
  }
}

// The W_UK product for few tokens: workgroup (head h, 64 outputs), wave ->
// 16 outputs; each lane loads its 4 W_UK chunks and 8 q^nope chunks at once
// and the 16x16 tiles are written straight from the accumulators.
constexpr int AR_J = 64;  // outputs per workgroup

__global__ __launch_bounds__(256) void absorb_rows_kernel(const bf16_t* __restrict__ qn, int64_t T, int H,
                                                          const bf16_t* __restrict__ wuk, void* q,
                                                          int64_t q_stride, int q_f32) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int h = blockIdx.x / (D_C / AR_J), jb = blockIdx.x % (D_C / AR_J);
  const int j = AR_J * jb + 16 * w + col;
  const int64_t tok0 = (int64_t)blockIdx.y * PR_TOK;
  uint4 b[4], a[2][4];
#pragma unroll
  for (int st = 0; st < 4; ++st) b[st] = load8_bf16(wuk + ((int64_t)h * D_C + j) * D_V + 32 * st + 8 * kg);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int64_t t = min(tok0 + 16 * mt + col, T - 1);
#pragma unroll
    for (int st = 0; st < 4; ++st) a[mt][st] = load8_bf16(qn + (t * H + h) * D_V + 32 * st + 8 * kg);
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) acc = mfma16x16x32(a[mt][st], b[st], acc);
    // acc[r] = q_abs[token 16 mt + 4 kg + r][output j]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = tok0 + 16 * mt + 4 * kg + r;
      if (t >= T) continue;
      const int64_t o = t * q_stride + (int64_t)h * D_ROW + j;
      if (q_f32) reinterpret_cast<float*>(q)[o] = acc[r];
      else reinterpret_cast<bf16_t*>(q)[o] = (bf16_t)f2bf(acc[r]);
    }
  }
}

// The absorption for more than a few tokens, q_abs[t, h, n] = sum_k
// qn[t, h, k] W_UK[h][n][k]: per token and head 256 B read, 1 KB (bf16)
// written, 131 kflop, so it is bound by the output stores. Persistent
// workgroups, each bound to one head h for the whole launch (grid = H x
// groups, heads fastest, so the workgroups of a head sit on one XCD and share
// its L2 copy of W_UK[h]). Wavefront w keeps output columns [128 w, 128 w +
// 128) of W_UK[h] in registers as the A operands of 32x32x16 MFMA (four
// 32-row blocks x 8 k-steps, 128 VGPRs). The workgroup's q^nope rows (tiles
// of 32 tokens, 8 KB) reach LDS by direct loads, a whole batch of tiles at
// once, and are read back as B operands; the stores of every tile then
// stream out with no wait on a load in between. A wave turns its 32 x 128
// results around in a private LDS area so that each store instruction writes
// whole 256-byte (bf16) or 512-byte (f32) row pieces of a few tokens rather
// than 32 bytes of each of 32 tokens.
constexpr int AS_TOK = 32;                 // tokens per tile (the N extent of a 32x32 block)
constexpr int AS_TILE = AS_TOK * D_V * 2;  // 8,192 bytes
// tiles resident at once: the q^nope batch and the four waves' staging areas
// fill the 160 KB of LDS
template <typename TQ> constexpr int as_batch() { return sizeof(TQ) == 2 ? 16 : 12; }
template <typename TQ> constexpr int as_stage() { return AS_TOK * 128 * (int)sizeof(TQ); }  // per wave

// k slots: lane half hf, k-step ks, element e hold k = 64 hf + 8 ks + e, so a
// lane's 8 operands of one W_UK row lie in one 128-byte line. LDS rows (a
// token's q^nope, or a token's 128 staged results) keep 16-byte chunk c at
// slot c ^ (row & 15), so 16 lanes that touch one chunk of 16 rows, or 16
// chunks of one row, cover all 64 banks once. Row i of a 32-row A block is
// output column 16 ((i >> 2) & 1) + 4 (i >> 3) + (i & 3) of the block: the 16
// results a lane holds are then 16 consecutive columns.
template <typename TQ>
__global__ __launch_bounds__(256) void absorb_stream_kernel(const bf16_t* __restrict__ qn, int64_t T, int H,
                                                            const bf16_t* __restrict__ wuk, TQ* __restrict__ q,
                                                            int64_t q_stride, int n_groups) {
  constexpr int NB = as_batch<TQ>(), SZ = (int)sizeof(TQ);
  constexpr int RP = 128 * SZ;      // bytes per staged row (the wave's 128 results of a token)
  constexpr int CH = RP / 16;        // 16-byte chunks per staged row (16 or 32)
  __shared__ __align__(16) unsigned char ql[NB * AS_TILE + 4 * as_stage<TQ>()];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x % H, grp = blockIdx.x / H;
  const int64_t n_tiles = (T + AS_TOK - 1) / AS_TOK;
  if (grp >= n_tiles) return;
  const int64_t my_tiles = (n_tiles - 1 - grp) / n_groups + 1;  // tiles grp, grp + n_groups, ...
  const int i = lane & 31, hf = lane >> 5;

  uint4 wa[4][8];
  {
    const int n = 128 * w + 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    const bf16_t* wr = wuk + ((int64_t)h * D_C + n) * D_V + 64 * hf;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) wa[jb][ks] = load8_bf16(wr + 32 * jb * D_V + 8 * ks);
  }

  const uint32_t lds0 = lds_off(ql);
  unsigned char* stage = ql + NB * AS_TILE + w * as_stage<TQ>();
  for (int64_t b0 = 0; b0 < my_tiles; b0 += NB) {
    const int nb = (int)min((int64_t)NB, my_tiles - b0);
    if (b0 > 0) barrier();  // every wave is done with the previous batch
    // tile u of the batch: wave w loads slots [128 w, 128 w + 128) (token rows
    // 8 w .. 8 w + 7); rows past T repeat row T - 1 and are never stored
    for (int u = 0; u < nb; ++u) {
      const int64_t tok0 = (grp + (b0 + u) * n_groups) * AS_TOK;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ii = 2 * w + j, P = 64 * ii + lane, r = P >> 4, c = (P & 15) ^ (r & 15);
        const int64_t t = min(tok0 + r, T - 1);
        dma16(qn + (t * H + h) * D_V + 8 * c, lds0 + (uint32_t)(u * AS_TILE) + 1024u * (uint32_t)ii);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();
    for (int u = 0; u < nb; ++u) {
      const unsigned char* tb = ql + u * AS_TILE + 256 * i;
      uint4 bq[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) bq[ks] = *reinterpret_cast<const uint4*>(tb + 16 * ((8 * hf + ks) ^ (i & 15)));
      f32x16_t acc[4];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[jb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) acc[jb] = mfma32x32x16(wa[jb][ks], bq[ks], acc[jb]);
      // acc[jb][r] = q_abs[token tok0 + i][128 w + 32 jb + 16 hf + r]: into
      // staged row i, chunks (2 jb + hf) SZ + k, k < SZ, one 16-byte store
      // each (the wave's own area; its LDS operations run in order, so no
      // barrier is needed)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = acc[jb][r];
#pragma unroll
        for (int k = 0; k < SZ; ++k) {
          TQ* p = reinterpret_cast<TQ*>(stage + RP * i + 16 * (((2 * jb + hf) * SZ + k) ^ (i & 15)));
          if constexpr (SZ == 2) store8(p, v + 8 * k);
          else store4(p, v + 4 * k);
        }
      }
      // rows to global memory: lane -> token 64 / CH j + lane / CH, chunk lane % CH
      const int64_t tok0 = (grp + (b0 + u) * n_groups) * AS_TOK;
#pragma unroll
      for (int j = 0; j < CH / 2; ++j) {
        const int t = (64 / CH) * j + lane / CH, c = lane % CH;
        const uint4 val = *reinterpret_cast<const uint4*>(stage + RP * t + 16 * (c ^ (t & 15)));
        if (tok0 + t < T)
          *reinterpret_cast<uint4*>(q + (tok0 + t) * q_stride + (int64_t)h * D_ROW + 128 * w + c * (16 / SZ)) = val;
      }
    }
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
  if (T <= PR_MAX_T && d % (32 * PR_WAVES) == 0) {
    const unsigned chunks = (unsigned)((T + PR_TOK - 1) / PR_TOK);
    hipLaunchKernelGGL(proj_rows_kernel, dim3((unsigned)(D_C / PR_COLS + 12 * H + 4), chunks),
                       dim3(64 * PR_WAVES), 0, stream, pa, (int)(q_dtype == LCA_F32));
    hipLaunchKernelGGL(absorb_rows_kernel, dim3((unsigned)(H * (D_C / AR_J)), chunks), dim3(256), 0, stream,
                       (const bf16_t*)qn, T, H, (const bf16_t*)w_uk, q, q_stride, (int)(q_dtype == LCA_F32));
    return hipGetLastError();
  }
  const int64_t pb_n = (T + PB_BM - 1) / PB_BM * pb_columns(H);
  const dim3 gb((unsigned)(8 * ((pb_n + 7) / 8)));
  // 256-wide tiles once they fill most of the chip; below that the 128-wide
  // tiles keep more CUs busy
  const bool big = pb_n >= 224;
  if (big) {
    if (q_dtype == LCA_BF16) hipLaunchKernelGGL(proj_big_kernel<bf16_t>, gb, dim3(64 * PB_WAVES), 0, stream, pa);
    else hipLaunchKernelGGL(proj_big_kernel<float>, gb, dim3(64 * PB_WAVES), 0, stream, pa);
  } else {
    if (q_dtype == LCA_BF16) hipLaunchKernelGGL(proj_kernel<bf16_t>, g1, dim3(256), 0, stream, pa);
    else hipLaunchKernelGGL(proj_kernel<float>, g1, dim3(256), 0, stream, pa);
  }
  const int64_t as_tiles = (T + AS_TOK - 1) / AS_TOK;
  const int64_t as_fill = as_tiles < 256 / H ? as_tiles : 256 / H;  // one workgroup per CU
  const int as_groups = as_fill > 1 ? (int)as_fill : 1;
  const dim3 gs((unsigned)(as_groups * H));
  if (q_dtype == LCA_BF16)
    hipLaunchKernelGGL(absorb_stream_kernel<bf16_t>, gs, dim3(256), 0, stream, (const bf16_t*)qn, T, H,
                       (const bf16_t*)w_uk, (bf16_t*)q, q_stride, as_groups);
  else
    hipLaunchKernelGGL(absorb_stream_kernel<float>, gs, dim3(256), 0, stream, (const bf16_t*)qn, T, H,
                       (const bf16_t*)w_uk, (float*)q, q_stride, as_groups);
  return hipGetLastError();
}

}  // namespace lca
