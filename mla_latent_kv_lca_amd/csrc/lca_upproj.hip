// Per-head value up-projection out[t, h, :] = o_latent[t, h, :] @ W_UV[h],
// gfx950. MLA caches only the latent and projects it back to each head's
// value space at compute time ("新一代开源大模型架构演进与注意力机制深度对比解析",
// 三.1); with absorbed attention that projection is applied once to the
// attention output.
//
// Large T, bf16 o_latent (prefill): up_stream_kernel below. Large T, f32
// o_latent (the decode workspace of a batch above 64 sequences): a workgroup
// of 4 wavefronts computes 64 tokens x 128 outputs of one head (16 tokens per
// wave, eight 16x16 output tiles). W_UV[h] streams through LDS in four
// 128-row k-slices; the k-major rows are turned into MFMA operands with the
// same row-fragment + half-word shuffle used for the value product of
// attention. o_latent fragments come straight from global memory.
#include "lca_device.h"
#include "lca_internal.h"
#include "lca_stream.h"
#include "lca_up_rows.h"

#include <algorithm>
#include <type_traits>

namespace lca {

constexpr int UP_TOK = 64;         // tokens per workgroup
constexpr int UP_KS = 128;         // k rows of W per LDS slice
constexpr int UP_WROW = D_V + 8;   // bf16 per LDS row of W (272 bytes)

template <typename TO, typename TW, typename TY>
__global__ __launch_bounds__(256) void up_proj_kernel(const TO* __restrict__ x, int64_t T, int H,
                                                      const TW* __restrict__ wuv,
                                                      TY* __restrict__ y) {
  __shared__ __align__(16) bf16_t wl[UP_KS * UP_WROW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int h = blockIdx.y;
  const int64_t tok0 = (int64_t)blockIdx.x * UP_TOK + 16 * w;
  const int64_t my_tok = tok0 + col;  // A-operand row of this lane
  const bool row_ok = my_tok < T;
  const TO* xr = x + (my_tok * H + h) * D_C;
  const TW* wh = wuv + (int64_t)h * D_C * D_V;

  f32x4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < D_C; k0 += UP_KS) {
    __syncthreads();
    // stage W[h][k0 .. k0+128)[0..128) (2048 chunks of 8, 8 per thread)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 4, c8 = q & 15;
      *reinterpret_cast<uint4*>(wl + row * UP_WROW + 8 * c8) =
          load8_bf16(wh + (int64_t)(k0 + row) * D_V + 8 * c8);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < UP_KS / 32; ++ks) {
      const uint4 a = row_ok ? load8_bf16(xr + k0 + 32 * ks + 8 * kg) : make_uint4(0u, 0u, 0u, 0u);
      uint4 R[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        R[kk] = *reinterpret_cast<const uint4*>(wl + (32 * ks + 8 * kg + kk) * UP_WROW + 8 * col);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int wi = c >> 1;
        uint4 bop;
        if (c & 1) {
          bop.x = hi_pair(u4_get(R[0], wi), u4_get(R[1], wi));
          bop.y = hi_pair(u4_get(R[2], wi), u4_get(R[3], wi));
          bop.z = hi_pair(u4_get(R[4], wi), u4_get(R[5], wi));
          bop.w = hi_pair(u4_get(R[6], wi), u4_get(R[7], wi));
        } else {
          bop.x = lo_pair(u4_get(R[0], wi), u4_get(R[1], wi));
          bop.y = lo_pair(u4_get(R[2], wi), u4_get(R[3], wi));
          bop.z = lo_pair(u4_get(R[4], wi), u4_get(R[5], wi));
          bop.w = lo_pair(u4_get(R[6], wi), u4_get(R[7], wi));
        }
        // D[token 4kg + r][n-col] with n = 8 col + c
        acc[c] = mfma16x16x32(a, bop, acc[c]);
      }
    }
  }
  // acc[c][r] = out[tok0 + 4kg + r][h][8 col + c]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t t = tok0 + 4 * kg + r;
    if (t < T) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = acc[c][r];
      store8(y + (t * H + h) * D_V + 8 * col, v);
    }
  }
}

// Large T with a bf16 latent: persistent workgroups, each bound to one head h.
// A wavefront keeps its 32 output columns of W_UV[h] (512 x 32 bf16) in
// registers as the A operand of v_mfma_f32_32x32x16_bf16 for the whole launch;
// the latent rows of 32 tokens at a time (one 1 KB row per token) stream from
// HBM straight into LDS (a ring of three tiles, two in flight while the third
// is read) and are read back as the B operand, so every latent byte crosses
// HBM once and W_UV is read once per workgroup. Rows are stored with a
// 1040-byte pitch: the 32 rows read by one fragment then start 4 banks apart.
constexpr int US_TOK = 32;                        // tokens per tile (N extent of a 32x32 block)
constexpr int US_PITCH = 2 * D_C + 16;            // LDS bytes per latent row
constexpr int US_TILE = US_TOK * US_PITCH;        // 33,280 bytes
constexpr int US_ROWS_PER_WAVE = US_TOK / 4;      // DMA row loads per wave per tile
constexpr int US_AHEAD = 4;                       // B fragments in flight per wave

// NBUF tiles resident per workgroup (NBUF - 1 in flight while one is used).
// Measured at 131,072 tokens x 16 heads: 2 tiles and two workgroups per CU
// 495 us, 3 or 4 tiles and one workgroup per CU 452 / 456 us.
template <int NBUF> constexpr int us_wg_per_cu() { return NBUF == 2 ? 2 : 1; }
constexpr int US_NBUF = 3;

template <int NBUF, typename TW, typename TY>
__global__ __launch_bounds__(256, us_wg_per_cu<NBUF>()) void up_stream_kernel(
    const bf16_t* __restrict__ x, int64_t T, int H, const TW* __restrict__ wuv, TY* __restrict__ y, int n_groups) {
  __shared__ __align__(16) unsigned char xl[NBUF * US_TILE];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x % H, grp = blockIdx.x / H;
  const int64_t n_tiles = (T + US_TOK - 1) / US_TOK;
  if (grp >= n_tiles) return;
  const int64_t my_tiles = (n_tiles - 1 - grp) / n_groups + 1;  // tiles grp, grp + n_groups, ...

  // Row i of this wave's 32-row block is output column
  // n = 32 w + 16 ((i >> 2) & 1) + 4 (i >> 3) + (i & 3): the 16 results a lane
  // holds (rows 8 (r / 4) + 4 (lane / 32) + r % 4) are then the 16 consecutive
  // columns 32 w + 16 (lane / 32) + r.
  // W_UV[h] passes through LDS in two halves of 256 k-rows (dense 256-byte
  // rows); each k-major fragment is assembled by two transposed reads. In a
  // 16-lane group, lane 4 j + a points at row j of the 4-row block and at the
  // 4 columns the receiving lanes 4 a .. 4 a + 3 need.
  const int i = lane & 31, half = lane >> 5;
  const int pa = lane & 3, pj = (lane >> 2) & 3;
  const int pcol = 32 * w + 16 * (pa & 1) + 4 * (pa >> 1) + 8 * ((lane >> 4) & 1);
  const TW* wh = wuv + (int64_t)h * D_C * D_V;
  bf16_t* wl = reinterpret_cast<bf16_t*>(xl);
  uint4 wa[D_C / 16];
#pragma unroll
  for (int hk = 0; hk < 2; ++hk) {
    if (hk) __syncthreads();
    Raw8<TW> st[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) st[c] = raw8_load(wh + (int64_t)hk * (D_C / 2) * D_V + 8 * (threadIdx.x + 256 * c));
#pragma unroll
    for (int c = 0; c < 16; ++c) *reinterpret_cast<uint4*>(wl + 8 * (threadIdx.x + 256 * c)) = raw8_bf16(st[c]);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < D_C / 32; ++s) {
      const bf16_t* p = wl + (16 * s + 8 * half + pj) * D_V + pcol;
      const uint2 lo = lds_read_tr4(p), hi = lds_read_tr4(p + 4 * D_V);
      wa[16 * hk + s] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  __syncthreads();  // the W_UV staging area becomes the latent ring

  const uint32_t lds0 = lds_off(xl);
  // Rows of tile u: wave w loads rows 8 w .. 8 w + 7 (one 1 KB row per load;
  // rows past T repeat row T - 1 and are never stored).
  auto issue = [&](int64_t u) {
    const int64_t tile = grp + u * n_groups;
    const uint32_t dst = lds0 + (uint32_t)(u % NBUF) * US_TILE;
#pragma unroll
    for (int q = 0; q < US_ROWS_PER_WAVE; ++q) {
      const int r = US_ROWS_PER_WAVE * w + q;
      const int64_t t = min(tile * US_TOK + r, T - 1);
      dma16_nt(x + (t * H + h) * D_C + 8 * lane, dst + r * US_PITCH);
    }
  };
#pragma unroll
  for (int u = 0; u < NBUF; ++u)
    if (u < my_tiles) issue(u);

  static_assert(US_ROWS_PER_WAVE == 8 && NBUF <= 4, "vmcnt immediates assume 8 loads per tile");
  for (int64_t u = 0; u < my_tiles; ++u) {
    // this wave's loads of tile u are done once at most `newer` later tiles
    // (8 loads each) are in flight; stores issued in between only make the
    // wait longer
    const int64_t newer = min((int64_t)NBUF - 1, my_tiles - 1 - u);
    if (newer >= 3) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (newer == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (newer == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();
    const unsigned char* b = xl + (u % NBUF) * US_TILE + i * US_PITCH + 16 * half;
    // B fragments read US_AHEAD steps ahead of their product; the fences keep
    // the compiler from hoisting all 32 reads (which would spill W).
    f32x16_t a0 = {}, a1 = {};
    uint4 bq[US_AHEAD];
#pragma unroll
    for (int s = 0; s < US_AHEAD; ++s) bq[s] = *reinterpret_cast<const uint4*>(b + 32 * s);
#pragma unroll
    for (int s = 0; s < D_C / 16; ++s) {
      const uint4 cur = bq[s % US_AHEAD];
      if (s + US_AHEAD < D_C / 16) bq[s % US_AHEAD] = *reinterpret_cast<const uint4*>(b + 32 * (s + US_AHEAD));
      if (s & 1) a1 = mfma32x32x16(wa[s], cur, a1);
      else a0 = mfma32x32x16(wa[s], cur, a0);
      __builtin_amdgcn_sched_barrier(0);
    }
    barrier();  // every wave is done with this buffer
    const int64_t t = (grp + u * n_groups) * US_TOK + i;
    if (t < T) {
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = a0[r] + a1[r];
      TY* o = y + (t * H + h) * D_V + 32 * w + 16 * half;
      store8(o, v);
      store8(o + 8, v + 8);
    }
    if (u + NBUF < my_tiles) issue(u + NBUF);
  }
}

template <typename TO, typename TW>
static void launch_up_w(int y_dtype, dim3 grid, hipStream_t st, const void* x, int64_t T, int H,
                        const void* w, void* y) {
  if (T <= UP_SMALL_T) {  // few rows (decode): W_UV streamed once per XCD, see lca_up_rows.h
    launch_up_rows<RowsFromLatent<TO>, TW>(RowsFromLatent<TO>{(const TO*)x}, T, H, w, y, y_dtype, st);
    return;
  }
  if constexpr (std::is_same<TO, bf16_t>::value) {
    constexpr int NB = US_NBUF;
    const int64_t n_tiles = (T + US_TOK - 1) / US_TOK;
    const int n_groups = (int)std::max<int64_t>(1, std::min<int64_t>(n_tiles, 256 * us_wg_per_cu<NB>() / H));
    const dim3 g((unsigned)(n_groups * H));
    if (y_dtype == LCA_BF16)
      hipLaunchKernelGGL((up_stream_kernel<NB, TW, bf16_t>), g, dim3(256), 0, st, (const bf16_t*)x, T, H,
                         (const TW*)w, (bf16_t*)y, n_groups);
    else
      hipLaunchKernelGGL((up_stream_kernel<NB, TW, float>), g, dim3(256), 0, st, (const bf16_t*)x, T, H,
                         (const TW*)w, (float*)y, n_groups);
    return;
  }
  if (y_dtype == LCA_BF16)
    hipLaunchKernelGGL((up_proj_kernel<TO, TW, bf16_t>), grid, dim3(256), 0, st, (const TO*)x, T, H, (const TW*)w, (bf16_t*)y);
  else
    hipLaunchKernelGGL((up_proj_kernel<TO, TW, float>), grid, dim3(256), 0, st, (const TO*)x, T, H, (const TW*)w, (float*)y);
}

hipError_t launch_up_proj(const void* o_latent, int o_dtype, int64_t T, int H, const void* w_uv,
                          int w_dtype, void* out, int out_dtype, hipStream_t stream) {
  dim3 grid((unsigned)((T + UP_TOK - 1) / UP_TOK), (unsigned)H);
  if (o_dtype == LCA_BF16) {
    if (w_dtype == LCA_BF16) launch_up_w<bf16_t, bf16_t>(out_dtype, grid, stream, o_latent, T, H, w_uv, out);
    else launch_up_w<bf16_t, float>(out_dtype, grid, stream, o_latent, T, H, w_uv, out);
  } else {
    if (w_dtype == LCA_BF16) launch_up_w<float, bf16_t>(out_dtype, grid, stream, o_latent, T, H, w_uv, out);
    else launch_up_w<float, float>(out_dtype, grid, stream, o_latent, T, H, w_uv, out);
  }
  return hipGetLastError();
}

}  // namespace lca
