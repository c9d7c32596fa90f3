// Decode attention over a condensed latent cache, gfx950.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// 整体框架 (representatives concatenated with the local window, then standard
// attention). In absorbed MLA form every head's key is the shared 576-wide
// cached row and its value the row's 512-wide latent, so the H heads of one
// sequence form a 16-row (per head block) by entries product, like MQA.
//
// decode_kernel: one workgroup of 4 wavefronts per (split, sequence, head
// block). The split's entries stream through LDS in tiles of 32. Wave w owns
// latent columns [128w, 128w + 128) and RoPE columns [16w, 16w + 16): it forms
// the partial scores S^T = K Q^T over its columns on the matrix cores
// (16x16x32 / 16x16x16 bf16), the four partials are summed through LDS in a
// fixed order, every wave runs the same online softmax, and each wave
// accumulates the value product for its own 128 columns (16x16x32 bf16,
// fp32 accumulators). The cost per entry is 34,816 flop on 1,152 bytes,
// above what the fp32 vector units could sustain at HBM rate, hence MFMA.
// Partial (unnormalised output, running max, running sum) go to the
// caller's workspace; merge_kernel combines the splits in split order.
#include "lca_tile.h"

namespace lca {

constexpr int SX_ROW = 36;  // floats per head row of the score exchange (32 + pad)

template <typename TQ, typename TC>
__global__ __launch_bounds__(NT, 2) void decode_kernel(
    const TQ* __restrict__ q, int64_t q_seq, Seg reps, int64_t m, Seg raw, int64_t raw_begin,
    int64_t n_entries, int per_tiles, int S, float scale_log2, int H, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ o_final, float* __restrict__ lse_final) {
  __shared__ __align__(16) bf16_t tile[TILE * LDS_ROW];
  __shared__ __align__(16) float sx[4][HB][SX_ROW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int s = blockIdx.x, b = blockIdx.y, hg = blockIdx.z, HG = gridDim.z;

  EntrySrc<TC> src;
  src.init(reps, raw, b, m, raw_begin);
  const int64_t e_begin = (int64_t)s * per_tiles * TILE;
  const int64_t e_end = min(n_entries, e_begin + (int64_t)per_tiles * TILE);
  const int n_tiles = e_end > e_begin ? (int)((e_end - e_begin + TILE - 1) / TILE) : 0;

  // this wave's query fragments: head col of the block, its k columns
  const TQ* qh = q + (int64_t)b * q_seq + (int64_t)(hg * HB + col) * D_ROW;
  uint4 qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qa[ks] = load8_bf16(qh + 128 * w + 32 * ks + 8 * kg);
  const uint2 qr = load4_bf16(qh + D_C + 16 * w + 4 * kg);

  f32x4_t o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  uint4 buf[CH_PER_T];
  if (n_tiles > 0) tile_load(src, e_begin, e_end, buf, tid);
  for (int t = 0; t < n_tiles; ++t) {
    const int64_t e0 = e_begin + (int64_t)t * TILE;
    __syncthreads();  // the previous tile is no longer read
    tile_store(tile, buf, tid);
    __syncthreads();
    if (t + 1 < n_tiles) tile_load(src, e0 + TILE, e_end, buf, tid);

    // partial S^T over this wave's columns, two 16-entry blocks
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
      const bf16_t* rowp = tile + (16 * eb + col) * LDS_ROW;
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(*reinterpret_cast<const uint4*>(rowp + 128 * w + 32 * ks + 8 * kg),
                           qa[ks], acc);
      // the RoPE columns go to their own accumulator: a 16x16x16 product that
      // takes a 16x16x32 result as its accumulator lost that result here
      const f32x4_t accr = mfma16x16x16(*reinterpret_cast<const uint2*>(rowp + D_C + 16 * w + 4 * kg),
                                        qr, f32x4_t{0.f, 0.f, 0.f, 0.f});
      *reinterpret_cast<f32x4_t*>(&sx[w][col][16 * eb + 4 * kg]) = acc + accr;  // S[h=col][e]
    }
    __syncthreads();

    float z[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4_t acc = *reinterpret_cast<const f32x4_t*>(&sx[0][col][16 * half + 4 * kg]);
#pragma unroll
      for (int ww = 1; ww < 4; ++ww)
        acc += *reinterpret_cast<const f32x4_t*>(&sx[ww][col][16 * half + 4 * kg]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t e = e0 + 16 * half + 4 * kg + r;
        z[4 * half + r] = (e < e_end) ? acc[r] * scale_log2 : -INFINITY;
      }
    }
    uint4 pb;
    const float corr = softmax_update(z, m_run, l_run, pb);
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] *= corr;
    pv_slab(tile, 128 * w, kg, col, pb, o);
  }

  // o[c][r] = O[head col][128w + 32kg + 8r + c]
  const int head = hg * HB + col;
  const int dbase = 128 * w + 32 * kg;
  if (S == 1) {
    const float inv = 1.0f / l_run;
    float* dst = o_final + ((int64_t)b * H + head) * D_C + dbase;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = o[c][r] * inv;
      store8(dst + 8 * r, v);
    }
    if (lse_final != nullptr && w == 0 && kg == 0)
      lse_final[(int64_t)b * H + head] = (m_run + log2f(l_run)) * 0.69314718055994530942f;
  } else {
    const int64_t slot = (((int64_t)b * HG + hg) * S + s) * HB + col;
    float* dst = part_o + slot * D_C + dbase;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = o[c][r];
      store8(dst + 8 * r, v);
    }
    if (w == 0 && kg == 0) {
      part_ml[slot * 2 + 0] = m_run;
      part_ml[slot * 2 + 1] = l_run;
    }
  }
}

// Combine S split partials of one (sequence, head) for 128 output columns:
// o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, in split order.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml, int S,
                                                    int H, float* __restrict__ o,
                                                    float* __restrict__ lse) {
  const int dchunk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int HG = H / HB, hg = head / HB, hh = head % HB;
  const int t = threadIdx.x;
  const int64_t slot0 = ((int64_t)b * HG + hg) * S;  // slot(s) = (slot0 + s) * HB + hh
  __shared__ float red[256];
  __shared__ float4 acc_sh[8][32];

  float mx = -INFINITY;
  for (int s = t; s < S; s += 256) mx = fmaxf(mx, part_ml[((slot0 + s) * HB + hh) * 2]);
  red[t] = mx;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (t < k) red[t] = fmaxf(red[t], red[t + k]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float ls = 0.f;
  for (int s = t; s < S; s += 256) {
    const float* ml = part_ml + ((slot0 + s) * HB + hh) * 2;
    ls += exp2f(ml[0] - M) * ml[1];
  }
  red[t] = ls;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (t < k) red[t] += red[t + k];
    __syncthreads();
  }
  const float Ltot = red[0];

  const int ph = t >> 5, c4 = t & 31;
  const int d = 128 * dchunk + 4 * c4;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = ph; s < S; s += 8) {
    const int64_t slot = (slot0 + s) * HB + hh;
    const float wgt = exp2f(part_ml[slot * 2] - M);
    const float4 v = *reinterpret_cast<const float4*>(part_o + slot * D_C + d);
    a.x = fmaf(wgt, v.x, a.x); a.y = fmaf(wgt, v.y, a.y);
    a.z = fmaf(wgt, v.z, a.z); a.w = fmaf(wgt, v.w, a.w);
  }
  acc_sh[ph][c4] = a;
  __syncthreads();
  if (ph == 0) {
    float4 r = acc_sh[0][c4];
#pragma unroll
    for (int p = 1; p < 8; ++p) {
      const float4 v = acc_sh[p][c4];
      r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
    }
    const float inv = 1.0f / Ltot;
    *reinterpret_cast<float4*>(o + ((int64_t)b * H + head) * D_C + d) =
        make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
  }
  if (lse != nullptr && dchunk == 0 && t == 0)
    lse[(int64_t)b * H + head] = (M + log2f(Ltot)) * 0.69314718055994530942f;
}

DecodeSplit decode_split(int B, int HG, int64_t n_entries) {
  const int64_t n_tiles = (n_entries + TILE - 1) / TILE;
  const int64_t seqs = (int64_t)B * HG;
  int64_t cap = (DEC_TARGET_BLOCKS + seqs - 1) / seqs;
  if (cap < 1) cap = 1;
  int64_t s0 = n_tiles < cap ? n_tiles : cap;
  if (s0 < 1) s0 = 1;
  const int64_t per = (n_tiles + s0 - 1) / s0;
  int64_t S = per > 0 ? (n_tiles + per - 1) / per : 1;
  if (S < 1) S = 1;
  return DecodeSplit{(int)S, (int)(per > 0 ? per : 1)};
}

size_t decode_workspace_bytes(int B, int HG, int S) {
  if (S <= 1) return 0;
  const size_t slots = (size_t)B * HG * S * HB;
  return slots * D_C * sizeof(float) + slots * 2 * sizeof(float);
}

template <typename TQ, typename TC>
static void launch_dec_t(dim3 grid, hipStream_t st, const void* q, int64_t q_seq, Seg reps,
                         int64_t m, Seg raw, int64_t raw_begin, int64_t n, int per, int S,
                         float sl2, int H, float* po, float* pml, float* of, float* lf) {
  hipLaunchKernelGGL((decode_kernel<TQ, TC>), grid, dim3(NT), 0, st, (const TQ*)q, q_seq, reps, m,
                     raw, raw_begin, n, per, S, sl2, H, po, pml, of, lf);
}

hipError_t launch_decode(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                         const lca_latent_t& reps, int64_t m, const lca_latent_t& raw,
                         int64_t raw_begin, int64_t raw_end, float sm_scale, float* o_latent,
                         float* lse, void* workspace, hipStream_t stream) {
  const int HG = H / HB;
  const int64_t n = m + (raw_end - raw_begin);
  const DecodeSplit sp = decode_split(B, HG, n);
  float* po = nullptr;
  float* pml = nullptr;
  if (sp.S > 1) {
    const size_t slots = (size_t)B * HG * sp.S * HB;
    po = static_cast<float*>(workspace);
    pml = po + slots * D_C;
  }
  const float sl2 = sm_scale * 1.44269504088896340736f;
  const Seg rs = to_seg(reps), ws = to_seg(raw);
  const int cdt = (m > 0) ? reps.dtype : raw.dtype;
  dim3 grid((unsigned)sp.S, (unsigned)B, (unsigned)HG);
  if (q_dtype == LCA_BF16) {
    if (cdt == LCA_BF16) launch_dec_t<bf16_t, bf16_t>(grid, stream, q, q_seq_stride, rs, m, ws, raw_begin, n, sp.per_tiles, sp.S, sl2, H, po, pml, o_latent, lse);
    else launch_dec_t<bf16_t, float>(grid, stream, q, q_seq_stride, rs, m, ws, raw_begin, n, sp.per_tiles, sp.S, sl2, H, po, pml, o_latent, lse);
  } else {
    if (cdt == LCA_BF16) launch_dec_t<float, bf16_t>(grid, stream, q, q_seq_stride, rs, m, ws, raw_begin, n, sp.per_tiles, sp.S, sl2, H, po, pml, o_latent, lse);
    else launch_dec_t<float, float>(grid, stream, q, q_seq_stride, rs, m, ws, raw_begin, n, sp.per_tiles, sp.S, sl2, H, po, pml, o_latent, lse);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || sp.S == 1) return err;
  hipLaunchKernelGGL(merge_kernel, dim3(4, (unsigned)H, (unsigned)B), dim3(256), 0, stream, po, pml,
                     sp.S, H, o_latent, lse);
  return hipGetLastError();
}

}  // namespace lca
