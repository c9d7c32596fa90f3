// Per-head value up-projection out[t, h, :] = o_latent[t, h, :] @ W_UV[h],
// gfx950. MLA caches only the latent and projects it back to each head's
// value space at compute time ("新一代开源大模型架构演进与注意力机制深度对比解析",
// 三.1); with absorbed attention that projection is applied once to the
// attention output.
//
// Large T: a workgroup of 4 wavefronts computes 64 tokens x 128 outputs of one head
// (16 tokens per wave, eight 16x16 output tiles). W_UV[h] streams through
// LDS in four 128-row k-slices; the k-major rows are turned into MFMA
// operands with the same row-fragment + half-word shuffle used for the value
// product of attention. o_latent fragments come straight from global memory.
#include "lca_device.h"
#include "lca_internal.h"
#include "lca_up_rows.h"

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

template <typename TO, typename TW>
static void launch_up_w(int y_dtype, dim3 grid, hipStream_t st, const void* x, int64_t T, int H,
                        const void* w, void* y) {
  if (T <= UP_SMALL_T) {  // few rows (decode): W_UV streamed once per XCD, see lca_up_rows.h
    launch_up_rows<RowsFromLatent<TO>, TW>(RowsFromLatent<TO>{(const TO*)x}, T, H, w, y, y_dtype, st);
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
