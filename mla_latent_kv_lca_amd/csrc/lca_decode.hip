// Decode attention over a condensed latent cache, gfx950.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// 整体框架 (representatives concatenated with the local window, then standard
// attention). In absorbed MLA form every head's key is the shared 576-wide
// cached row and its value the row's 512-wide latent, so the H heads of one
// sequence form a 16-row (per head block) by entries product, like MQA.
//
// Kernels:
//  decode_kernel         bf16 rows packed as [c_KV ++ k_R]: HBM -> LDS ring by
//                        direct loads, one workgroup per CU (details below).
//  decode_kernel_staged  any strides / f32 rows: register-staged 32-entry tiles.
//  merge_kernel          combines split-K partial results in split order.
#include <mutex>

#include "lca_stream.h"
#include "lca_up_rows.h"

namespace lca {

constexpr int SX_ROW = 36;                     // floats per head row of the staged score exchange
constexpr int DNW = 4;                         // wavefronts per decode workgroup
constexpr int DNT = 64 * DNW;                  // threads per decode workgroup
constexpr int DT = STILE;                      // entries per split-planning tile
constexpr int WT = 16;                         // entries per wave tile
constexpr int WSLOT = 2;                       // LDS slots per wavefront
constexpr int WT_ELEMS = WT * D_ROW;           // 9,216 bf16 = 18,432 bytes
constexpr int WT_DMA = WT * (D_ROW / 8) / 64;  // 18 direct loads per wave tile

// decode_kernel: one workgroup of 4 wavefronts per (split, sequence, head
// block), one workgroup per CU. A sequence's entries are cut into 16-entry
// wave tiles, dealt round robin over the 4 S wavefronts of its S splits
// (wave w of split s takes tiles 4 s + w + 4 S k); each wavefront runs its own online softmax over its own entries for all 16
// heads and all 576 columns, so there is no cross-wave exchange (and no
// barrier) per tile. Its tiles stream from HBM straight into its own two LDS
// slots (global_load_lds, 16 bytes per lane, 18 loads per tile, completion
// tracked with its own vmcnt); a slot is refilled as soon as its tile's value
// product is done. Per tile the wavefront
//   forms S^T = K Q^T for its 16 entries (18 MFMA 16x16x32 in two chains,
//   the 16 heads' queries in registers as the B operand), and
//   accumulates O^T += V^T P^T over all 512 latent columns (32 MFMA
//   16x16x16; P comes straight from the score registers, V^T from transposed
//   LDS reads, ds_read_b64_tr_b16).
// The four wavefronts' states are merged once, at the end, in wave order.
// The cost per entry is 34,816 flop on 1,152 bytes, more than the fp32
// vector units sustain at HBM rate, hence the matrix cores.
// With S > 1 splits per sequence the workgroup writes its merged (O, max,
// sum) to the workspace and a second kernel combines the splits in split order.
//
// Tile layout: the dense rows of lca_stream.h (chunk c of row r at c ^ swz(r)),
// so the 16 rows x 1 chunk of a K fragment and the 4 rows x 2 chunks of a
// transposed V^T read both touch distinct LDS bank groups.
// Reductions over the four 16-lane rows holding one head (lanes col + 16 k):
// v_permlane16_swap / v_permlane32_swap exchange lane halves in registers;
// both results of a swap are combined, so every lane gets the same value.
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct loads (non-temporal: a decode step reads each row once, and a
// model's cache over all layers far exceeds the Infinity Cache) of wave tile
// entries [e0, e0 + WT) into `slot`: LDS position
// P = 64 i + lane holds chunk (P % 72) ^ swz(row) of tile row row = P / 72.
// Full tiles inside one segment use a uniform row base plus per-lane
// offsets; the tile that straddles the representative / raw boundary and the
// last, partial tile compute each row, reloading the last valid row past
// e_end (those logits are masked, so any finite row will do).
__device__ __forceinline__ void wave_tile_dma(const DmaSrc& src, int64_t e0, int64_t e_end,
                                              const bf16_t* slot, int lane,
                                              const uint32_t (&off)[WT_DMA]) {
  const uint32_t base = lds_off(slot);
  if (e0 + WT <= e_end && (e0 + WT <= src.m || e0 >= src.m)) {
    const char* b0 = e0 < src.m ? src.rep + e0 * src.tok : src.raw + (e0 - src.m) * src.tok;
    dma16_rows<1024u, true>(b0, off, base);
  } else {
    const int valid = (int)min((int64_t)WT, e_end - e0);
    for (int i = 0; i < WT_DMA; ++i) {
      const int P = 64 * i + lane, row = P / (D_ROW / 8);
      const int c = (P - row * (D_ROW / 8)) ^ swz(row);
      const int64_t e = e0 + min(row, valid - 1);
      const char* p = e < src.m ? src.rep + e * src.tok : src.raw + (e - src.m) * src.tok;
      dma16_nt(p + 16 * c, base + 1024u * i);
    }
  }
}
// wait until at most `newer` wave tiles issued after the one wanted are in flight
__device__ __forceinline__ void wait_wave_tile(int newer) {
  static_assert(WSLOT == 2 && WT_DMA == 18, "vmcnt immediates assume 2 slots of 18 loads");
  if (newer >= 1) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// A sequence's attended entries as 16-entry wave tiles. DenseTiles: entries
// [0, n) = representative rows [0, m) ++ raw rows, in one token stride.
struct DenseTiles {
  DmaSrc src;
  int64_t n;
  __device__ __forceinline__ int64_t count() const { return (n + WT - 1) / WT; }
  __device__ __forceinline__ int valid(int64_t u) const { return (int)min((int64_t)WT, n - u * WT); }
  __device__ __forceinline__ void dma(int64_t u, const bf16_t* slot, int lane, const uint32_t (&off)[WT_DMA]) const {
    wave_tile_dma(src, u * WT, n, slot, lane, off);
  }
};

// PagedTiles: ceil(m / 16) tiles of dense representative rows, then the raw
// rows [raw_begin, raw_end) of a paged cache (rows of token t in page
// table[t / P], row t % P), 16 tokens per tile from raw_begin on. A tile
// touches at most two pages (P is a multiple of 16); its page indices are
// wave-uniform loads. Rows past the valid ones reload the last valid row
// (their logits are masked).
struct PagedTiles {
  const char* rep;        // this sequence's representative rows
  const char* pages;      // page pool
  const int32_t* table;   // this sequence's block table
  int64_t tok;            // row stride in bytes (representatives and pages)
  int64_t m, raw_begin, raw_end, R;  // R = representative tiles
  int P;                  // rows per page
  __device__ __forceinline__ int64_t count() const { return R + (raw_end - raw_begin + WT - 1) / WT; }
  __device__ __forceinline__ int valid(int64_t u) const {
    return u < R ? (int)min((int64_t)WT, m - u * WT) : (int)min((int64_t)WT, raw_end - raw_begin - (u - R) * WT);
  }
  __device__ __forceinline__ void dma(int64_t u, const bf16_t* slot, int lane, const uint32_t (&off)[WT_DMA]) const {
    const uint32_t base = lds_off(slot);
    const int v = valid(u);
    if (u < R) {
      const char* b0 = rep + u * WT * tok;
      if (v == WT) {
        dma16_rows<1024u, true>(b0, off, base);
      } else {
        for (int i = 0; i < WT_DMA; ++i) {
          const int Q = 64 * i + lane, row = Q / (D_ROW / 8), c = (Q - row * (D_ROW / 8)) ^ swz(row);
          dma16_nt(b0 + min(row, v - 1) * tok + 16 * c, base + 1024u * i);
        }
      }
      return;
    }
    const int64_t t0 = raw_begin + (u - R) * WT, pg0 = t0 / P, pg1 = (t0 + v - 1) / P;
    const int64_t p0 = table[__builtin_amdgcn_readfirstlane((int)pg0)];
    const int64_t p1 = table[__builtin_amdgcn_readfirstlane((int)pg1)];
    if (v == WT && pg0 == pg1) {
      dma16_rows<1024u, true>(pages + (p0 * P + (t0 - pg0 * P)) * tok, off, base);
    } else {
      for (int i = 0; i < WT_DMA; ++i) {
        const int Q = 64 * i + lane, row = Q / (D_ROW / 8), c = (Q - row * (D_ROW / 8)) ^ swz(row);
        const int64_t t = t0 + min(row, v - 1), pg = t / P;
        const int64_t page = pg == pg0 ? p0 : p1;
        dma16_nt(pages + (page * P + (t - pg * P)) * tok + 16 * c, base + 1024u * i);
      }
    }
  }
};

template <typename TQ, class Tiles>
__device__ __forceinline__ void decode_body(bf16_t (&ring)[DNW][WSLOT][WT_ELEMS], const TQ* __restrict__ q,
                                            int64_t q_seq, const Tiles& tiles, int64_t tok_b, int S,
                                            float scale_log2, int H, float* __restrict__ part_o,
                                            float* __restrict__ part_ml, float* __restrict__ o_final,
                                            float* __restrict__ lse_final) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, col = lane & 15;
  const int s = blockIdx.x, b = blockIdx.y, hg = blockIdx.z, HG = gridDim.z;

  // the sequence's wave tiles are dealt round robin over the S x 4
  // wavefronts of its splits: this wave takes u0 + ustep k, k < n_mine, so at
  // any time the sequence's wavefronts read one narrow window of its entries
  const int64_t n_wt = tiles.count();
  const int64_t u0 = w + (int64_t)DNW * s, ustep = (int64_t)DNW * S;
  const int n_mine = n_wt > u0 ? (int)((n_wt - 1 - u0) / ustep + 1) : 0;

  uint32_t off[WT_DMA];
#pragma unroll
  for (int i = 0; i < WT_DMA; ++i) {
    const int P = 64 * i + lane, row = P / (D_ROW / 8);
    off[i] = (uint32_t)(row * tok_b) + 16u * ((P - row * (D_ROW / 8)) ^ swz(row));
  }
  auto issue = [&](int k) { tiles.dma(u0 + ustep * k, &ring[w][k % WSLOT][0], lane, off); };
  // lane-constant element offsets inside a wave tile.
  // Score product, k-step ks: lane (kg, col) reads row col, chunk 4 ks + kg,
  // at kb[ks & 1] + 64 (ks >> 1) (swz only flips the low three chunk bits).
  const int swc = swz(col);
  const int kb[2] = {8 * (col * (D_ROW / 8) + (kg ^ swc)), 8 * (col * (D_ROW / 8) + ((4 + kg) ^ swc))};

  // The queries (B operand of head col, 18 k-steps of 32 columns). bf16: the
  // 16 query rows travel like a tile, by direct loads into slot 1, with tile
  // 0 right behind them; the wave waits for the queries only (the splits of
  // a sequence share them, so they usually come from L2 before tile 0),
  // copies them into registers, and slot 1 then takes tile 1 while tile 0 may
  // still be in flight.
  // f32: register loads (rounded to bf16), waited for before any tile is in
  // flight (requested behind the tiles, they would only arrive with them).
  uint4 qa[18];
  const TQ* qh = q + (int64_t)b * q_seq + (int64_t)(hg * HB) * D_ROW;
  const int last_row = min(HB, H - hg * HB) - 1;  // rows past it repeat it (never stored)
  if constexpr (sizeof(TQ) == 2) {
    const uint32_t qbase = lds_off(&ring[w][1][0]);
#pragma unroll
    for (int i = 0; i < WT_DMA; ++i) {
      const int P = 64 * i + lane, row = P / (D_ROW / 8);
      dma16(qh + min(row, last_row) * D_ROW + 8 * ((P - row * (D_ROW / 8)) ^ swz(row)), qbase + 1024u * i);
    }
    if (n_mine > 0) {
      issue(0);
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");  // the queries (tile 0 may still be in flight)
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const bf16_t* qt = &ring[w][1][0];
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qa[ks] = *reinterpret_cast<const uint4*>(qt + kb[ks & 1] + 64 * (ks >> 1));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (n_mine > 1) issue(1);
  } else {
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qa[ks] = load8_bf16(qh + min(col, last_row) * D_ROW + 32 * ks + 8 * kg);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) retire(qa[ks]);
#pragma unroll
    for (int k = 0; k < WSLOT; ++k)
      if (k < n_mine) issue(k);
  }
  // Value product, column tile ct (latent columns 16 ct .. 16 ct + 15): a
  // transposed read gives lane (kg, col) the values of rows 4 kg .. 4 kg + 3
  // in column 16 ct + col -- the A operand of V^T -- when the 16 lanes of row
  // group kg point at rows 4 kg + col / 4, columns 16 ct + 4 (col % 4) .. + 3;
  // that address is vb[ct & 3] + 64 (ct >> 2).
  const int vr = 4 * kg + (col >> 2), swv = swz(vr);
  int vb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vb[j] = 8 * (vr * (D_ROW / 8) + ((2 * j + ((col >> 1) & 1)) ^ swv)) + 4 * (col & 1);

  f32x4_t o[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Scores of wave tile k (log2 units, rows past the tile's valid ones masked); returns their
  // per-head maximum.
  // The tile's V^T operands (all 32 transposed reads), read right after the
  // score products so that their latency hides under the softmax and the
  // slot can take its next tile before the value products.
  uint2 vf[32];
  auto scores = [&](int k, float (&z)[4]) -> float {
    const int valid = tiles.valid(u0 + ustep * k);
    wait_wave_tile(min(n_mine - 1 - k, WSLOT - 1));
    const bf16_t* tile = &ring[w][k % WSLOT][0];
    f32x4_t sa = f32x4_t{0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
    for (int ks = 0; ks < 18; ks += 2) {
      sa = mfma16x16x32(*reinterpret_cast<const uint4*>(tile + kb[0] + 64 * (ks >> 1)), qa[ks], sa);
      sb = mfma16x16x32(*reinterpret_cast<const uint4*>(tile + kb[1] + 64 * (ks >> 1)), qa[ks + 1], sb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) vf[ct] = lds_read_tr4(tile + vb[ct & 3] + 64 * (ct >> 2));
    __builtin_amdgcn_sched_barrier(0);
    const f32x4_t sc = sa + sb;  // S[entry 4 kg + r][head col]
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = sc[r] * scale_log2;
    if (valid < WT) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * kg + r >= valid) z[r] = -INFINITY;
    }
    // per head: lanes col, col + 16, col + 32, col + 48
    return xor32_max(xor16_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]))));
  };
  // Probabilities relative to the running max, their sum, the slot's next
  // tile (wave tile k + WSLOT, once the V^T reads are done), and the value
  // product O^T += V^T P^T (32 column tiles).
  auto accumulate = [&](int k, const float (&z)[4]) {
    // a wave with no visible entry yet keeps m_run = -inf: its p must be 0
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(z[r] - m_ref);
    l_run += xor32_sum(xor16_sum((p[0] + p[1]) + (p[2] + p[3])));
    const uint2 pb = make_uint2(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]));
    if (k + WSLOT < n_mine) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(k + WSLOT);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
      // o[ct][r] = O[head col][16 ct + 4 kg + r]
      o[ct] = mfma16x16x16(vf[ct], pb, o[ct]);
    }
  };
  // Online softmax with a lazy rescale: the inner loop runs while the running
  // max stays within LAZY_LOG2 of every new score, so the accumulators are
  // touched only by the MFMA there; a tile that raises it leaves the loop,
  // rescales, and the loop resumes after it.
  int k = 0;
  while (k < n_mine) {
    float z[4], tmax = 0.f;
    for (; k < n_mine; ++k) {
      tmax = scores(k, z);
      if (__builtin_amdgcn_ballot_w64(tmax > m_run + LAZY_LOG2) != 0) break;
      accumulate(k, z);
    }
    if (k >= n_mine) break;
    const float m_new = fmaxf(m_run, tmax);
    const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= corr;
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] *= corr;
    m_run = m_new;
    accumulate(k, z);
    ++k;
  }

  // merge the four wavefronts through LDS (the ring is free now):
  // [w][head][EXR] then [w][head][2]; rows padded by 4 floats so that the
  // heads of one access fall on different LDS banks
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  barrier();
  constexpr int EXR = D_C + 4;
  float* ex = reinterpret_cast<float*>(&ring[0][0][0]);
  float* exml = ex + DNW * HB * EXR;
#pragma unroll
  for (int ct = 0; ct < 32; ++ct)
    *reinterpret_cast<f32x4_t*>(ex + (w * HB + col) * EXR + 16 * ct + 4 * kg) = o[ct];
  if (kg == 0) {
    exml[(w * HB + col) * 2 + 0] = m_run;
    exml[(w * HB + col) * 2 + 1] = l_run;
  }
  barrier();
  // wave w finalises latent columns [128 w, 128 w + 128) of every head: lane
  // -> head col, 32 columns starting at 128 w + 32 kg; the four states are
  // added in wave order
  float mw[DNW], M = -INFINITY;
#pragma unroll
  for (int i = 0; i < DNW; ++i) {
    mw[i] = exml[(i * HB + col) * 2];
    M = fmaxf(M, mw[i]);
  }
  float Lsum = 0.f, acc[32];
  const int d0 = 128 * w + 32 * kg;
#pragma unroll
  for (int i = 0; i < DNW; ++i) {
    const float wt = mw[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[i] - M);
    Lsum = i == 0 ? wt * exml[(i * HB + col) * 2 + 1] : fmaf(wt, exml[(i * HB + col) * 2 + 1], Lsum);
    const float4* pi = reinterpret_cast<const float4*>(ex + (i * HB + col) * EXR + d0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 v = pi[j];
      acc[4 * j + 0] = i == 0 ? wt * v.x : fmaf(wt, v.x, acc[4 * j + 0]);
      acc[4 * j + 1] = i == 0 ? wt * v.y : fmaf(wt, v.y, acc[4 * j + 1]);
      acc[4 * j + 2] = i == 0 ? wt * v.z : fmaf(wt, v.z, acc[4 * j + 2]);
      acc[4 * j + 3] = i == 0 ? wt * v.w : fmaf(wt, v.w, acc[4 * j + 3]);
    }
  }
  const int head = hg * HB + col;
  if (S == 1) {
    if (head >= H) return;
    const float inv = 1.0f / Lsum;
    float* dst = o_final + ((int64_t)b * H + head) * D_C + d0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = acc[8 * i + c] * inv;
      store8(dst + 8 * i, v);
    }
    if (lse_final != nullptr && w == 0 && kg == 0)
      lse_final[(int64_t)b * H + head] = (M + __log2f(Lsum)) * 0.69314718055994530942f;
    return;
  }
  const int64_t slot = (((int64_t)b * HG + hg) * S + s) * HB + col;
  float* dst = part_o + slot * D_C + d0;
#pragma unroll
  for (int i = 0; i < 4; ++i) store8(dst + 8 * i, acc + 8 * i);
  if (w == 0 && kg == 0) {
    part_ml[slot * 2 + 0] = M;
    part_ml[slot * 2 + 1] = Lsum;
  }
}

template <typename TQ>
__global__ __launch_bounds__(DNT) void decode_kernel(
    const TQ* __restrict__ q, int64_t q_seq, DmaSrc src0, int64_t rep_seq_b, int64_t raw_seq_b,
    int64_t n_entries, int S, float scale_log2, int H, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ o_final, float* __restrict__ lse_final) {
  __shared__ __align__(16) bf16_t ring[DNW][WSLOT][WT_ELEMS];  // 147,456 bytes
  DenseTiles tiles;
  tiles.src = src0;
  tiles.src.rep += (int64_t)blockIdx.y * rep_seq_b;
  tiles.src.raw += (int64_t)blockIdx.y * raw_seq_b;
  tiles.n = n_entries;
  decode_body<TQ>(ring, q, q_seq, tiles, src0.tok, S, scale_log2, H, part_o, part_ml, o_final, lse_final);
}

// Ragged batch over a paged cache: per-sequence representative count and raw
// range from device arrays.
template <typename TQ>
__global__ __launch_bounds__(DNT) void decode_paged_kernel(
    const TQ* __restrict__ q, int64_t q_seq, const char* __restrict__ rep, int64_t rep_seq_b,
    const int32_t* __restrict__ seq_m, const char* __restrict__ pages, const int32_t* __restrict__ table,
    int64_t table_stride, int page_rows, const int32_t* __restrict__ seq_raw_begin,
    const int32_t* __restrict__ seq_raw_end, int64_t tok_b, int S, float scale_log2, int H,
    float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ o_final,
    float* __restrict__ lse_final) {
  __shared__ __align__(16) bf16_t ring[DNW][WSLOT][WT_ELEMS];  // 147,456 bytes
  const int b = blockIdx.y;
  PagedTiles tiles;
  tiles.rep = rep + (int64_t)b * rep_seq_b;
  tiles.pages = pages;
  tiles.table = table + (int64_t)b * table_stride;
  tiles.tok = tok_b;
  tiles.P = page_rows;
  tiles.m = seq_m[b];
  tiles.raw_begin = seq_raw_begin[b];
  tiles.raw_end = seq_raw_end[b];
  tiles.R = (tiles.m + WT - 1) / WT;
  decode_body<TQ>(ring, q, q_seq, tiles, tok_b, S, scale_log2, H, part_o, part_ml, o_final, lse_final);
}

// Register-staged variant for f32 caches (rounded to bf16 as they are staged
// into LDS); the bf16 path above copies rows into LDS without conversion.
template <typename TQ, typename TC>
__global__ __launch_bounds__(NT) void decode_kernel_staged(
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

  // this wave's query fragments: head col of the block (rows past the last
  // head repeat it and are never stored), its k columns
  const TQ* qh = q + (int64_t)b * q_seq + (int64_t)(hg * HB + min(col, H - 1 - hg * HB)) * D_ROW;
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
    if (head >= H) return;
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

// Combine the S split partials of a (sequence, head):
//   o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s,
// always in split order. Few splits: one thread per 4 output columns.
__global__ __launch_bounds__(256) void merge_small_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml, int S,
                                                          int B, int H, float* __restrict__ o,
                                                          float* __restrict__ lse) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)B * H * (D_C / 4)) return;
  const int c4 = (int)(gid % (D_C / 4));
  const int64_t bh = gid / (D_C / 4);
  const int head = (int)(bh % H), b = (int)(bh / H);
  const int HG = head_blocks(H), hg = head / HB, hh = head % HB;
  float M, L;
  const float4 v = merge_cols4(part_o, part_ml, S, ((int64_t)b * HG + hg) * S, hh, c4, M, L);
  reinterpret_cast<float4*>(o + ((int64_t)b * H + head) * D_C)[c4] = v;
  if (lse != nullptr && c4 == 0) lse[(int64_t)b * H + head] = (M + log2f(L)) * 0.69314718055994530942f;
}

// Many splits (one long sequence): workgroup per (32 columns, head, sequence),
// 32 split phases x 8 threads of 4 columns; phase partials added in order.
// Many splits (one long sequence): workgroup (32 latent columns, head,
// sequence); thread (phase p, 4 columns) takes splits p, p + 32, ...: all of
// its loads (up to MERGE_UNROLL splits) are issued at once, the max and then
// the weighted sums are formed from registers in split order, and the 32
// phase partials are added in phase order.
constexpr int MERGE_UNROLL = 8;  // splits per thread held in registers (S <= 256)
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml, int S,
                                                    int H, float* __restrict__ o,
                                                    float* __restrict__ lse) {
  const int dchunk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int HG = head_blocks(H), hg = head / HB, hh = head % HB;
  const int t = threadIdx.x, ph = t >> 3, c4 = t & 7;
  const int64_t slot0 = ((int64_t)b * HG + hg) * S;  // slot(s) = (slot0 + s) * HB + hh
  const int d = 32 * dchunk + 4 * c4;
  __shared__ float red[2][32];
  __shared__ float4 acc_sh[32][8];

  float2 ml[MERGE_UNROLL];
  float4 v[MERGE_UNROLL];
#pragma unroll
  for (int i = 0; i < MERGE_UNROLL; ++i) {
    const int s = ph + 32 * i;
    if (s < S) {
      const int64_t slot = (slot0 + s) * HB + hh;
      ml[i] = reinterpret_cast<const float2*>(part_ml)[slot];
      v[i] = *reinterpret_cast<const float4*>(part_o + slot * D_C + d);
    } else {
      ml[i] = make_float2(-INFINITY, 0.f);
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < MERGE_UNROLL; ++i) mx = fmaxf(mx, ml[i].x);
  for (int s = ph + 32 * MERGE_UNROLL; s < S; s += 32) mx = fmaxf(mx, part_ml[((slot0 + s) * HB + hh) * 2]);
  if (c4 == 0) red[0][ph] = mx;
  __syncthreads();
  float M = red[0][0];
  for (int p = 1; p < 32; ++p) M = fmaxf(M, red[0][p]);
  float ls = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < MERGE_UNROLL; ++i) {
    const float wgt = ml[i].x == -INFINITY ? 0.f : exp2f(ml[i].x - M);
    ls = fmaf(wgt, ml[i].y, ls);
    a.x = fmaf(wgt, v[i].x, a.x); a.y = fmaf(wgt, v[i].y, a.y);
    a.z = fmaf(wgt, v[i].z, a.z); a.w = fmaf(wgt, v[i].w, a.w);
  }
  for (int s = ph + 32 * MERGE_UNROLL; s < S; s += 32) {  // beyond 256 splits (not produced by the planner)
    const int64_t slot = (slot0 + s) * HB + hh;
    const float ms = part_ml[slot * 2];
    const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
    ls = fmaf(wgt, part_ml[slot * 2 + 1], ls);
    const float4 u = *reinterpret_cast<const float4*>(part_o + slot * D_C + d);
    a.x = fmaf(wgt, u.x, a.x); a.y = fmaf(wgt, u.y, a.y);
    a.z = fmaf(wgt, u.z, a.z); a.w = fmaf(wgt, u.w, a.w);
  }
  if (c4 == 0) red[1][ph] = ls;
  acc_sh[ph][c4] = a;
  __syncthreads();
  if (ph == 0) {
    float Lt = red[1][0];
    float4 r = acc_sh[0][c4];
    for (int p = 1; p < 32; ++p) {
      Lt += red[1][p];
      const float4 u = acc_sh[p][c4];
      r.x += u.x; r.y += u.y; r.z += u.z; r.w += u.w;
    }
    const float inv = 1.0f / Lt;
    *reinterpret_cast<float4*>(o + ((int64_t)b * H + head) * D_C + d) =
        make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
    if (lse != nullptr && dchunk == 0 && c4 == 0)
      lse[(int64_t)b * H + head] = (M + log2f(Lt)) * 0.69314718055994530942f;
  }
}

DecodeSplit decode_split(int B, int HG, int64_t n_entries) {
  const int64_t n_tiles = (n_entries + DT - 1) / DT;
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

// workspace: [m, l: slots * 2][O: slots * 512], slots = B * HG * S * 16
size_t decode_workspace_bytes(int B, int HG, int S) {
  if (S <= 1) return 0;
  const size_t slots = (size_t)B * HG * S * HB;
  return slots * 2 * sizeof(float) + slots * D_C * sizeof(float);
}

static bool packed_rows(const lca_latent_t& t) {
  return t.c != nullptr && t.dtype == LCA_BF16 &&
         static_cast<const char*>(t.kr) == static_cast<const char*>(t.c) + 2 * D_C &&
         t.kr_tok_stride == t.c_tok_stride && t.kr_seq_stride == t.c_seq_stride;
}

// The attention kernel of one decode call; with sp.S > 1 it leaves split
// partials in the workspace (pml: [slots][2], po: [slots][512]).
static hipError_t decode_attention(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                                   const lca_latent_t& reps, int64_t m, const lca_latent_t& raw,
                                   int64_t raw_begin, int64_t raw_end, float sm_scale,
                                   float* o_latent, float* lse, const DecodeSplit& sp, float* po,
                                   float* pml, hipStream_t stream) {
  const int HG = head_blocks(H);
  const int64_t n = m + (raw_end - raw_begin);
  const float sl2 = sm_scale * 1.44269504088896340736f;
  dim3 grid((unsigned)sp.S, (unsigned)B, (unsigned)HG);
  const bool has_rep = m > 0, has_raw = raw_end > raw_begin;
  const int64_t tok = has_rep ? reps.c_tok_stride : raw.c_tok_stride;
  const bool fast = (!has_rep || packed_rows(reps)) && (!has_raw || packed_rows(raw)) &&
                    (!has_rep || !has_raw || reps.c_tok_stride == raw.c_tok_stride) &&
                    tok * 2 * DT < ((int64_t)1 << 31);
  if (fast) {
    DmaSrc src;
    src.rep = has_rep ? static_cast<const char*>(reps.c) : nullptr;
    src.raw = has_raw ? static_cast<const char*>(raw.c) + raw_begin * raw.c_tok_stride * 2 : nullptr;
    src.tok = tok * 2;
    src.m = m;
    const int64_t rep_seq_b = m > 0 ? reps.c_seq_stride * 2 : 0;
    const int64_t raw_seq_b = raw_end > raw_begin ? raw.c_seq_stride * 2 : 0;
    if (q_dtype == LCA_BF16)
      hipLaunchKernelGGL(decode_kernel<bf16_t>, grid, dim3(DNT), 0, stream, (const bf16_t*)q,
                         q_seq_stride, src, rep_seq_b, raw_seq_b, n, sp.S, sl2, H, po, pml, o_latent, lse);
    else
      hipLaunchKernelGGL(decode_kernel<float>, grid, dim3(DNT), 0, stream, (const float*)q,
                         q_seq_stride, src, rep_seq_b, raw_seq_b, n, sp.S, sl2, H, po, pml, o_latent, lse);
  } else {
    // general strides or f32 rows: register-staged kernel, 32-entry tiles
    const Seg rs = to_seg(reps), ws = to_seg(raw);
    const int cdt = (m > 0) ? reps.dtype : raw.dtype;
#define LCA_STAGED(TQ, TC)                                                                       \
  hipLaunchKernelGGL((decode_kernel_staged<TQ, TC>), grid, dim3(NT), 0, stream, (const TQ*)q,      \
                     q_seq_stride, rs, m, ws, raw_begin, n, sp.per_tiles, sp.S, sl2, H, po,        \
                     pml, o_latent, lse)
    if (q_dtype == LCA_BF16 && cdt == LCA_BF16) LCA_STAGED(bf16_t, bf16_t);
    else if (q_dtype == LCA_BF16) LCA_STAGED(bf16_t, float);
    else if (cdt == LCA_BF16) LCA_STAGED(float, bf16_t);
    else LCA_STAGED(float, float);
#undef LCA_STAGED
  }
  return hipGetLastError();
}

static void split_buffers(void* workspace, int B, int HG, const DecodeSplit& sp, float*& po, float*& pml) {
  po = pml = nullptr;
  if (sp.S > 1) {
    const size_t slots = (size_t)B * HG * sp.S * HB;
    pml = static_cast<float*>(workspace);
    po = pml + slots * 2;
  }
}

static void launch_merge(const DecodeSplit& sp, int B, int H, const float* po, const float* pml,
                         float* o_latent, float* lse, hipStream_t stream) {
  if (sp.S <= MERGE_SMALL_S) {
    const int64_t n = (int64_t)B * H * (D_C / 4);
    hipLaunchKernelGGL(merge_small_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       po, pml, sp.S, B, H, o_latent, lse);
  } else {
    hipLaunchKernelGGL(merge_kernel, dim3(D_C / 32, (unsigned)H, (unsigned)B), dim3(256), 0, stream,
                       po, pml, sp.S, H, o_latent, lse);
  }
}

hipError_t launch_decode(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                         const lca_latent_t& reps, int64_t m, const lca_latent_t& raw,
                         int64_t raw_begin, int64_t raw_end, float sm_scale, float* o_latent,
                         float* lse, void* workspace, hipStream_t stream) {
  const DecodeSplit sp = decode_split(B, head_blocks(H), m + (raw_end - raw_begin));
  float *po, *pml;
  split_buffers(workspace, B, head_blocks(H), sp, po, pml);
  hipError_t err = decode_attention(q, q_dtype, q_seq_stride, B, H, reps, m, raw, raw_begin, raw_end,
                                    sm_scale, o_latent, lse, sp, po, pml, stream);
  if (err != hipSuccess || sp.S == 1) return err;
  launch_merge(sp, B, H, po, pml, o_latent, lse, stream);
  return hipGetLastError();
}

// The attention kernel of one paged decode call; with sp.S > 1 it leaves
// split partials in the workspace.
static hipError_t decode_paged_attention(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                                         const lca_latent_t& reps, const int32_t* seq_m, const lca_paged_t& cache,
                                         const int32_t* seq_raw_begin, const int32_t* seq_raw_end,
                                         float sm_scale, float* o_latent, float* lse, const DecodeSplit& sp,
                                         float* po, float* pml, hipStream_t stream) {
  const int HG = head_blocks(H);
  const float sl2 = sm_scale * 1.44269504088896340736f;
  dim3 grid((unsigned)sp.S, (unsigned)B, (unsigned)HG);
  const char* rep = static_cast<const char*>(reps.c);
  const int64_t rep_seq_b = reps.c_seq_stride * 2, tok_b = cache.row_stride * 2;
  const char* pages = static_cast<const char*>(cache.pages);
  if (q_dtype == LCA_BF16)
    hipLaunchKernelGGL(decode_paged_kernel<bf16_t>, grid, dim3(DNT), 0, stream, (const bf16_t*)q, q_seq_stride,
                       rep, rep_seq_b, seq_m, pages, cache.block_table, cache.table_stride, cache.page_rows,
                       seq_raw_begin, seq_raw_end, tok_b, sp.S, sl2, H, po, pml, o_latent, lse);
  else
    hipLaunchKernelGGL(decode_paged_kernel<float>, grid, dim3(DNT), 0, stream, (const float*)q, q_seq_stride,
                       rep, rep_seq_b, seq_m, pages, cache.block_table, cache.table_stride, cache.page_rows,
                       seq_raw_begin, seq_raw_end, tok_b, sp.S, sl2, H, po, pml, o_latent, lse);
  return hipGetLastError();
}

hipError_t launch_decode_paged(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                               const lca_latent_t& reps, const int32_t* seq_m, const lca_paged_t& cache,
                               const int32_t* seq_raw_begin, const int32_t* seq_raw_end,
                               int64_t max_entries, float sm_scale, float* o_latent, float* lse,
                               void* workspace, hipStream_t stream) {
  const DecodeSplit sp = decode_split(B, head_blocks(H), max_entries);
  float *po, *pml;
  split_buffers(workspace, B, head_blocks(H), sp, po, pml);
  hipError_t err = decode_paged_attention(q, q_dtype, q_seq_stride, B, H, reps, seq_m, cache, seq_raw_begin,
                                          seq_raw_end, sm_scale, o_latent, lse, sp, po, pml, stream);
  if (err != hipSuccess || sp.S == 1) return err;
  launch_merge(sp, B, H, po, pml, o_latent, lse, stream);
  return hipGetLastError();
}

// The split merge (or the W_UV projection of the merged rows) after a
// decode attention kernel that left its partials in po / pml.
static hipError_t merge_and_up(const DecodeSplit& sp, int B, int H, float* po, float* pml, float* o_latent,
                               float* lse, const void* w_uv, int w_dtype, void* out, int out_dtype,
                               hipStream_t stream) {
  hipError_t err;
  if (sp.S == 1 || sp.S > MERGE_SMALL_S || B > UP_SMALL_T) {
    if (sp.S > 1) launch_merge(sp, B, H, po, pml, o_latent, lse, stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return launch_up_proj(o_latent, LCA_F32, B, H, w_uv, w_dtype, out, out_dtype, stream);
  }
  const RowsFromSplits rows{po, pml, sp.S, o_latent, lse};
  if (w_dtype == LCA_BF16) launch_up_rows<RowsFromSplits, bf16_t>(rows, B, H, w_uv, out, out_dtype, stream);
  else launch_up_rows<RowsFromSplits, float>(rows, B, H, w_uv, out, out_dtype, stream);
  return hipGetLastError();
}

hipError_t launch_decode_paged_up(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                                  const lca_latent_t& reps, const int32_t* seq_m, const lca_paged_t& cache,
                                  const int32_t* seq_raw_begin, const int32_t* seq_raw_end, int64_t max_entries,
                                  float sm_scale, float* o_latent, float* lse, const void* w_uv, int w_dtype,
                                  void* out, int out_dtype, void* workspace, hipStream_t stream) {
  const DecodeSplit sp = decode_split(B, head_blocks(H), max_entries);
  float *po, *pml;
  split_buffers(workspace, B, head_blocks(H), sp, po, pml);
  const hipError_t err = decode_paged_attention(q, q_dtype, q_seq_stride, B, H, reps, seq_m, cache, seq_raw_begin,
                                                seq_raw_end, sm_scale, o_latent, lse, sp, po, pml, stream);
  if (err != hipSuccess) return err;
  return merge_and_up(sp, B, H, po, pml, o_latent, lse, w_uv, w_dtype, out, out_dtype, stream);
}

hipError_t launch_decode_paged_up_step(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                                       const lca_latent_t& reps, int32_t* seq_m, const lca_paged_t& cache,
                                       int32_t* seq_raw_begin, int32_t* seq_raw_end, int64_t max_entries,
                                       float sm_scale, float* o_latent, float* lse, const void* w_uv, int w_dtype,
                                       void* out, int out_dtype, void* workspace, int64_t w, int g, void* q_ring,
                                       int64_t q_ring_seq_stride, int32_t* anchor, int64_t anchor_seq, int32_t* pos,
                                       int64_t* dst_row, hipStream_t stream) {
  const DecodeSplit sp = decode_split(B, head_blocks(H), max_entries);
  float *po, *pml;
  split_buffers(workspace, B, head_blocks(H), sp, po, pml);
  hipError_t err = decode_paged_attention(q, q_dtype, q_seq_stride, B, H, reps, seq_m, cache, seq_raw_begin,
                                          seq_raw_end, sm_scale, o_latent, lse, sp, po, pml, stream);
  if (err != hipSuccess) return err;
  if (B > UP_SMALL_T) {  // the projection takes the large-T kernel: the step is its own launch
    if ((err = merge_and_up(sp, B, H, po, pml, o_latent, lse, w_uv, w_dtype, out, out_dtype, stream)) != hipSuccess)
      return err;
    return launch_condense_step(cache, B, w, g, q, q_dtype, q_seq_stride, H, q_ring, q_ring_seq_stride, sm_scale,
                                reps, anchor, anchor_seq, seq_m, seq_raw_begin, seq_raw_end, pos, dst_row, stream);
  }
  int s_rows = sp.S;  // the rows the projection kernel reads: split partials (merged there) or merged rows
  if (sp.S > MERGE_SMALL_S) {
    launch_merge(sp, B, H, po, pml, o_latent, lse, stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    s_rows = 1;
  }
  return launch_up_rows_step(po, pml, s_rows, o_latent, lse, B, H, w_uv, w_dtype, out, out_dtype, cache, w, g, q,
                             q_dtype, q_seq_stride, q_ring, q_ring_seq_stride, sm_scale, reps, anchor, anchor_seq,
                             seq_m, seq_raw_begin, seq_raw_end, pos, dst_row, stream);
}

// ---- scratch for the entry point that allocates nothing
// Split-K partial results of mla_latent_attn_decode_up_noalloc live in this
// file-scope array instead of a caller workspace. Every GPU the library runs
// on holds its own copy until the process ends. In host code the name is
// only a stand-in: its device address comes from hipGetSymbolAddress, looked
// up once per device (with that device current) and kept here.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_up(const void* q, int q_dtype, int64_t q_seq_stride, int B, int H,
                            const lca_latent_t& reps, int64_t m, const lca_latent_t& raw,
                            int64_t raw_begin, int64_t raw_end, float sm_scale, float* o_latent,
                            float* lse, const void* w_uv, int w_dtype, void* out, int out_dtype,
                            void* workspace, hipStream_t stream) {
  const DecodeSplit sp = decode_split(B, head_blocks(H), m + (raw_end - raw_begin));
  float *po, *pml;
  split_buffers(workspace, B, head_blocks(H), sp, po, pml);
  const hipError_t err = decode_attention(q, q_dtype, q_seq_stride, B, H, reps, m, raw, raw_begin, raw_end,
                                          sm_scale, o_latent, lse, sp, po, pml, stream);
  if (err != hipSuccess) return err;
  return merge_and_up(sp, B, H, po, pml, o_latent, lse, w_uv, w_dtype, out, out_dtype, stream);
}

}  // namespace lca
