// Chunked prefill attention over a condensed latent cache, gfx950.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// 整体框架: each query attends to the representatives of the groups older
// than its window plus the uncompressed rows (causal within the window). The
// groups a chunk sees are fixed before the chunk starts, so one chunk is a
// causal flash-attention over [reps ++ raw rows] shared by all H heads.
//
// Workgroup = 4 wavefronts = 4 consecutive query tokens; a wave holds the 16
// heads of its token (heads fill the 16-row side of every 16x16 MFMA tile,
// since all heads share the same keys and values). Entry tiles of 32 rows
// stream through LDS once per workgroup; per tile a wave forms S^T = K Q^T
// over the full 576 columns (18 MFMA 16x16x32 per 16 entries, its queries in
// registers), runs the online softmax in registers (four lanes per head) and
// accumulates O for all 512 latent columns (32 MFMA 16x16x32 per tile).
// Workgroups are issued heaviest (latest tokens) first.
#include "lca_tile.h"

namespace lca {

constexpr int PF_TOK = 4;  // query tokens per workgroup (one per wave)

template <typename TQ, typename TC, typename TO>
__global__ __launch_bounds__(NT) void prefill_kernel(
    const TQ* __restrict__ q, int64_t q_tok, int64_t chunk_start, int C, int H, Seg reps,
    int64_t m, Seg raw, int64_t raw_begin, float scale_log2, TO* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ __align__(16) bf16_t tile[TILE * LDS_ROW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int nblk = gridDim.x;
  const int blk = nblk - 1 - (int)blockIdx.x;  // heavy blocks first
  const int hg = blockIdx.y;
  const int i_tok = blk * PF_TOK + w;            // chunk row of this wave
  const bool active = i_tok < C;
  const int i_last = min(blk * PF_TOK + PF_TOK, C) - 1;

  EntrySrc<TC> src;
  src.init(reps, raw, 0, m, raw_begin);
  // entries visible to chunk row i: m + (chunk_start + i - raw_begin + 1)
  const int64_t n_mine = m + (chunk_start + (active ? i_tok : i_last) - raw_begin + 1);
  const int64_t n_blk = m + (chunk_start + i_last - raw_begin + 1);
  const int n_tiles = (int)((n_blk + TILE - 1) / TILE);

  const TQ* qh = q + (int64_t)(active ? i_tok : i_last) * q_tok + (int64_t)(hg * HB + col) * D_ROW;
  uint4 qa[18];
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) qa[ks] = load8_bf16(qh + 32 * ks + 8 * kg);

  f32x4_t oacc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) oacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  uint4 buf[CH_PER_T];
  tile_load(src, 0, n_blk, buf, tid);
  for (int t = 0; t < n_tiles; ++t) {
    const int64_t e0 = (int64_t)t * TILE;
    __syncthreads();
    tile_store(tile, buf, tid);
    __syncthreads();
    if (t + 1 < n_tiles) tile_load(src, e0 + TILE, n_blk, buf, tid);

    float z[8];
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
      const bf16_t* rowp = tile + (16 * eb + col) * LDS_ROW + 8 * kg;
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        acc = mfma16x16x32(*reinterpret_cast<const uint4*>(rowp + 32 * ks), qa[ks], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t e = e0 + 16 * eb + 4 * kg + r;
        z[4 * eb + r] = (e < n_mine) ? acc[r] * scale_log2 : -INFINITY;
      }
    }
    uint4 pb;
    const float corr = softmax_update(z, m_run, l_run, pb);
#pragma unroll
    for (int c = 0; c < 32; ++c) oacc[c] *= corr;
#pragma unroll
    for (int slab = 0; slab < 4; ++slab) pv_slab(tile, 128 * slab, kg, col, pb, oacc + 8 * slab);
  }

  if (!active) return;
  // oacc[8 slab + c][r] = O[head col][128 slab + 32 kg + 8 r + c]
  const int head = hg * HB + col;
  const float inv = 1.0f / l_run;
  TO* dst = o + ((int64_t)i_tok * H + head) * D_C + 32 * kg;
#pragma unroll
  for (int slab = 0; slab < 4; ++slab) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = oacc[8 * slab + c][r] * inv;
      store8(dst + 128 * slab + 8 * r, v);
    }
  }
  if (lse != nullptr && kg == 0)
    lse[(int64_t)i_tok * H + head] = (m_run + log2f(l_run)) * 0.69314718055994530942f;
}

template <typename TQ, typename TC, typename TO>
static void launch_pf_t(dim3 grid, hipStream_t st, const void* q, int64_t q_tok, int64_t cs,
                        int C, int H, Seg reps, int64_t m, Seg raw, int64_t rb, float sl2, void* o,
                        float* lse) {
  hipLaunchKernelGGL((prefill_kernel<TQ, TC, TO>), grid, dim3(NT), 0, st, (const TQ*)q, q_tok, cs,
                     C, H, reps, m, raw, rb, sl2, (TO*)o, lse);
}

template <typename TQ, typename TC>
static void launch_pf_o(int o_dtype, dim3 grid, hipStream_t st, const void* q, int64_t q_tok,
                        int64_t cs, int C, int H, Seg reps, int64_t m, Seg raw, int64_t rb,
                        float sl2, void* o, float* lse) {
  if (o_dtype == LCA_BF16) launch_pf_t<TQ, TC, bf16_t>(grid, st, q, q_tok, cs, C, H, reps, m, raw, rb, sl2, o, lse);
  else launch_pf_t<TQ, TC, float>(grid, st, q, q_tok, cs, C, H, reps, m, raw, rb, sl2, o, lse);
}

hipError_t launch_prefill(const void* q, int q_dtype, int64_t q_tok_stride, int64_t chunk_start,
                          int C, int H, const lca_latent_t& reps, int64_t m,
                          const lca_latent_t& raw, int64_t raw_begin, float sm_scale,
                          void* o_latent, int o_dtype, float* lse, hipStream_t stream) {
  const float sl2 = sm_scale * 1.44269504088896340736f;
  const Seg rs = to_seg(reps), ws = to_seg(raw);
  const int cdt = raw.dtype;
  dim3 grid((unsigned)((C + PF_TOK - 1) / PF_TOK), (unsigned)(H / HB));
  if (q_dtype == LCA_BF16) {
    if (cdt == LCA_BF16) launch_pf_o<bf16_t, bf16_t>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, rs, m, ws, raw_begin, sl2, o_latent, lse);
    else launch_pf_o<bf16_t, float>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, rs, m, ws, raw_begin, sl2, o_latent, lse);
  } else {
    if (cdt == LCA_BF16) launch_pf_o<float, bf16_t>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, rs, m, ws, raw_begin, sl2, o_latent, lse);
    else launch_pf_o<float, float>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, rs, m, ws, raw_begin, sl2, o_latent, lse);
  }
  return hipGetLastError();
}

}  // namespace lca
