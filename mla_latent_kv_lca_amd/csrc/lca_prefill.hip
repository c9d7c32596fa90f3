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
#include <cfloat>
#include <type_traits>

#include "lca_stream.h"

namespace lca {


// Register-staged variant for strided or f32 rows, one token (16 rows) per wave.
template <typename TQ, typename TC, typename TO>
__global__ __launch_bounds__(NT) void prefill_kernel_staged(
    const TQ* __restrict__ q, int64_t q_tok, int64_t chunk_start, int C, int H, int lhb, Seg reps,
    int64_t m, Seg raw, int64_t raw_begin, float scale_log2, TO* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ __align__(16) bf16_t tile[TILE * LDS_ROW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int nblk = gridDim.x;
  const int blk = nblk - 1 - (int)blockIdx.x;  // heavy blocks first
  const int hg = blockIdx.y;
  // query row R = 16 w + col is (token R >> lhb, head R % Hb), Hb = 2^lhb =
  // min(H, 16) heads per block: 64 / Hb tokens per workgroup
  const int n_tok = 64 >> lhb, hmask = (1 << lhb) - 1;
  const int i_tok = blk * n_tok + ((16 * w + col) >> lhb);  // chunk row of this lane's query row
  const bool active = i_tok < C;
  const int i_last = min(blk * n_tok + n_tok, C) - 1;

  EntrySrc<TC> src;
  src.init(reps, raw, 0, m, raw_begin);
  // entries visible to chunk row i: m + (chunk_start + i - raw_begin + 1)
  const int64_t n_mine = m + (chunk_start + (active ? i_tok : i_last) - raw_begin + 1);
  const int64_t n_blk = m + (chunk_start + i_last - raw_begin + 1);
  const int n_tiles = (int)((n_blk + TILE - 1) / TILE);

  const TQ* qh = q + (int64_t)(active ? i_tok : i_last) * q_tok + (int64_t)(hg * HB + (col & hmask)) * D_ROW;
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
  // oacc[8 slab + c][r] = O[query row col][128 slab + 32 kg + 8 r + c]
  const int head = hg * HB + (col & hmask);
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

// prefill_kernel: the fast path for packed bf16 rows. Workgroup = 4
// wavefronts = 2 pairs; pair p holds 32 query rows (2 query tokens x 16
// heads; with Hb < 16 heads, as in grouped-query attention, 32 / Hb tokens x
// Hb heads), so every LDS fragment feeds a 32x32x16 MFMA. Entry tiles of 32 rows
// stream HBM -> LDS by direct loads into a 4-slot ring (two tiles in
// flight). Within a pair, wave k
//   forms the partial S^T = K Q^T over query columns [288 k, 288 k + 288)
//   (18 MFMA 32x32x16, those query columns in registers) and adds its
//   partner's partial read through LDS, so both waves hold identical scores
//   and run the same online softmax (two lanes per query row; the reference
//   max only moves when a row's max grows by more than 2^8, so the
//   accumulators are rarely rescaled), and
//   accumulates O^T += V^T P^T for latent columns [256 k, 256 k + 256)
//   (16 MFMA 32x32x16; P comes straight from the score registers, V^T from
//   transposed LDS reads).
// The tiles run as a software pipeline, so that the matrix cores never wait
// for the vector work of the same tile: iteration t issues the score
// products of tile t + 1 with the softmax of tile t spread between them
// (phase A), then the value products of tile t with the partial-score
// exchange, sum, mask and row max of tile t + 1 spread between them (phase
// B). Scheduling fences keep every slot's few vector instructions next to
// its matrix product. Causal masking is compiled only into the (at most two)
// tiles that cross the diagonal of the workgroup's rows.
constexpr int PBUF = 4;     // LDS ring depth (tiles): 4 x 36 KB + 16 KB exchange = 160 KB
constexpr int KF_RING = 6;  // score-product fragments in registers (read four products ahead)
constexpr int VF_AHEAD = 4; // value-product operands read this many products ahead
constexpr int VF_RING = VF_AHEAD + 1;

template <bool V> using bool_c = std::integral_constant<bool, V>;

template <typename TQ, typename TO, class Src>
__global__ __launch_bounds__(256) void prefill_kernel(
    const TQ* __restrict__ q, int64_t q_tok, int64_t chunk_start, int C, int H, int lhb, Src src,
    int64_t m, int64_t raw_begin, float scale_log2, TO* __restrict__ o, float* __restrict__ lse) {
  __shared__ __align__(16) bf16_t ring[PBUF][STILE_ELEMS];
  __shared__ __align__(16) f32x4_t sx[4][4][64];  // partial scores [wave][r / 4][lane]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = w >> 1, kh = w & 1;  // pair, column half
  const int h32 = lane >> 5, r32 = lane & 31;
  const int blk = (int)gridDim.x - 1 - (int)blockIdx.x;  // heavy workgroups first
  const int hg = blockIdx.y;
  // query row R = 32 pr + r32 of the workgroup is (token R >> lhb, head
  // R % Hb) with Hb = 2^lhb = min(H, 16) heads per block: 64 / Hb tokens
  const int n_tok = 64 >> lhb, hmask = (1 << lhb) - 1;
  const int tok0 = blk * n_tok;
  const int i_tok = tok0 + ((32 * pr + r32) >> lhb);  // chunk row of this lane's query row
  const bool active = i_tok < C;
  const int i_ld = active ? i_tok : C - 1;
  const int i_last = min(tok0 + n_tok, C) - 1;
  // entries visible to chunk row i: m + (chunk_start + i - raw_begin + 1)
  const int64_t vis0 = m + (chunk_start - raw_begin + 1);
  const int64_t n_blk = vis0 + i_last, n_min = vis0 + tok0, n_mine = vis0 + i_ld;
  const int n_tiles = (int)((n_blk + STILE - 1) / STILE);
  const int n_full = (int)(n_min / STILE);  // tiles every row of the workgroup sees whole

  uint32_t off[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    int row, col16;
    slot_rowcol(w, i, lane, row, col16);
    off[i] = (uint32_t)(row * src.tok) + 16u * col16;
  }
#pragma unroll
  for (int t = 0; t < PBUF - 1; ++t)
    if (t < n_tiles) tile_dma(src, (int64_t)t * STILE, n_blk, ring[t], w, lane, off);

  // Q^T operand: query row (token i_ld, head hg*16 + r32 % Hb), k = 288 kh + 16 ks + 8 h32 ..
  const TQ* qh = q + (int64_t)i_ld * q_tok + (int64_t)(hg * HB + (r32 & hmask)) * D_ROW + 288 * kh + 8 * h32;
  uint4 qf[18];
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) qf[ks] = load8_bf16(qh + 16 * ks);
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) retire(qf[ks]);  // wait here once, not inside the loop

  f32x16_t oacc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[c][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Value-product operands come from transposed LDS reads
  // (ds_read_b64_tr_b16): for column tile ct (32 latent columns) and entry
  // k-step kap, lane l (row group g = l / 16: h32 = g / 2, column half
  // rh = g % 2) needs V[entry][256 kh + 32 ct + 16 rh + l % 16] for the 8
  // entries that its P operand holds (16 kap + 4 h32 + 0..3, then + 8). Read a
  // gives the four entries 16 kap + 8 a + 4 h32 + 0..3 when the 16 lanes of
  // the group point at entry rows (l % 16) / 4 of that run, columns
  // 4 ((l % 16) % 4) .. + 3 of the 16-column half: the offsets below are
  // those addresses for ct = 0, kap = 0.
  // With e = 16 kap + 8 a + tr_row0 (swz(e) = swz(8 a + tr_row0)) and column
  // chunk x + 4 ct (x & 4 = 0), the position (x + 4 ct) ^ swz(e) splits into
  // (x ^ (swz & 3)) and 4 (ct ^ bit 2 of swz): per read a, two per-lane bases
  // (even / odd ct) plus constants.
  const int tr_row0 = 4 * h32 + ((lane & 15) >> 2);
  const int tr_col0 = 256 * kh + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int tr_off[2][2];  // [a][ct & 1], + 32 ct + 576 * 16 kap
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int row = 8 * a + tr_row0, sw = swz(row);
    const int base = 8 * (row * (D_ROW / 8) + ((tr_col0 >> 3) ^ (sw & 3))) + (tr_col0 & 7);
    tr_off[a][0] = base + 32 * (sw >> 2);
    tr_off[a][1] = base - 32 * (sw >> 2);
  }
  // Score-product operand, k-step f (query columns 288 kh + 16 f + 8 h32 ..):
  // chunk c = 36 kh + 2 f + h32 of row r32, at kq[f & 3] + 64 (f >> 2) (swz
  // only flips the low three chunk bits, so four per-lane bases cover all f).
  const int sw32 = swz(r32);
  int kq[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int F = jj + 2 * kh;
    kq[jj] = 8 * (r32 * (D_ROW / 8)) + 256 * kh + 64 * (F >> 2) + 8 * ((2 * (F & 3) + h32) ^ sw32);
  }
  auto kfrag = [&](const bf16_t* tile, int f) {
    return *reinterpret_cast<const uint4*>(tile + kq[f & 3] + 64 * (f >> 2));
  };
  // value-product operand j = 8 kap + ct of a tile
  auto vfrag = [&](const bf16_t* tile, int j) {
    const int kap = j >> 3, ct = j & 7;
    const bf16_t* pa = tile + 32 * ct + D_ROW * 16 * kap;
    const uint2 lo = lds_read_tr4(pa + tr_off[0][ct & 1]);
    const uint2 hi = lds_read_tr4(pa + tr_off[1][ct & 1]);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };

  float z[16];   // scores of the current tile, unscaled (-inf where masked)
  uint4 pb[2];   // its softmax weights as bf16, entry k-steps 0 and 1
  f32x16_t S, S2;  // partial scores of the next tile, two product chains (even / odd k-steps)
  uint4 vf[VF_RING];  // value-product operands, read VF_AHEAD products ahead

  // Phase A: score products of tile tn (QK, two independent accumulator
  // chains, so that no product waits for the previous one) and, spread
  // between them, the softmax of the current tile z (SM): p = 2^(scale z -
  // m_run), row sum into l_run, p packed to bf16 into pb. Also reads the
  // first VF_AHEAD value operands of the current tile tc for phase B (PV).
  auto phase_a = [&](auto qk, auto sm, auto pv, const bf16_t* tn, const bf16_t* tc) {
    constexpr bool QK = decltype(qk)::value, SM = decltype(sm)::value, PV = decltype(pv)::value;
    const float m_ref = m_run;
    float p[16], ps = 0.f;
    uint4 kf[KF_RING];
    if constexpr (QK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) { S[r] = 0.f; S2[r] = 0.f; }
#pragma unroll
      for (int f = 0; f < 4; ++f) kf[f] = kfrag(tn, f);
    }
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if constexpr (QK) {
        if (ks & 1) S2 = mfma32x32x16(kf[ks % KF_RING], qf[ks], S2);
        else S = mfma32x32x16(kf[ks % KF_RING], qf[ks], S);
        if (ks + 4 < 18) kf[(ks + 4) % KF_RING] = kfrag(tn, ks + 4);
      }
      if constexpr (SM) {
        if (ks < 16) {
          p[ks] = __builtin_amdgcn_exp2f(fmaf(z[ks], scale_log2, -m_ref));
          ps += p[ks];
          if (ks & 1) {
            const int k = ks >> 1;  // packed pair k of 8: entry k-step k / 4, word k % 4
            const uint32_t wd = pack_bf2(p[ks - 1], p[ks]);
            if ((k & 3) == 0) pb[k >> 2].x = wd;
            else if ((k & 3) == 1) pb[k >> 2].y = wd;
            else if ((k & 3) == 2) pb[k >> 2].z = wd;
            else pb[k >> 2].w = wd;
          }
        } else if (ks == 16) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
          l_run += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
      }
      if constexpr (PV) {  // the score fragments are all read by slot 13
        if (ks >= 18 - VF_AHEAD) vf[ks - (18 - VF_AHEAD)] = vfrag(tc, ks - (18 - VF_AHEAD));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Phase B: value products of tile tc (PV) and, spread between them, the
  // exchange of the partial scores of the next tile (XC): this wave's
  // partial written to LDS, a barrier, the partner's read back and added
  // (fp32 addition commutes, so both waves of the pair hold the same sums),
  // causally masked (MASKED, entries from en0), and the row max returned in
  // log2 units.
  auto phase_b = [&](auto pv, auto xc, auto masked, const bf16_t* tc, int64_t en0) -> float {
    constexpr bool PV = decltype(pv)::value, XC = decltype(xc)::value, MASKED = decltype(masked)::value;
    f32x4_t sp[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (PV) {
        const int kap = j >> 3, ct = j & 7;
        oacc[ct] = mfma32x32x16(vf[j % VF_RING], pb[kap], oacc[ct]);
        if (j + VF_AHEAD < 16) vf[(j + VF_AHEAD) % VF_RING] = vfrag(tc, j + VF_AHEAD);
      }
      if constexpr (XC) {
        if (j >= 2 && j < 6) {  // this wave's partial: the two chains added
          const int r4 = j - 2;
          sx[w][r4][lane] = f32x4_t{S[4 * r4] + S2[4 * r4], S[4 * r4 + 1] + S2[4 * r4 + 1],
                                    S[4 * r4 + 2] + S2[4 * r4 + 2], S[4 * r4 + 3] + S2[4 * r4 + 3]};
        }
        if (j == 7) barrier();  // both partials of the pair are in LDS
        if (j >= 8 && j < 12) sp[j - 8] = sx[w ^ 1][j - 8][lane];
        if (j >= 12) {
          const int r4 = j - 12;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * r4 + i;
            float v = (S[r] + S2[r]) + sp[r4][i];
            if constexpr (MASKED) {
              if (en0 + 8 * (r >> 2) + 4 * h32 + (r & 3) >= n_mine) v = -INFINITY;
            }
            z[r] = v;
            tmax = fmaxf(tmax, v);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (XC) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    return tmax * scale_log2;  // scale > 0, so the max commutes with it
  };
  // Lazy rescale: the reference max only moves when some row's new max
  // exceeds it by more than 2^LAZY_LOG2 (always on the first tile).
  auto rescale = [&](float tmax) {
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + LAZY_LOG2) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
      // one accumulator tile at a time (left to itself the compiler copies
      // all 128 accumulator registers out at once and spills)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        oacc[c] *= corr;
        __builtin_amdgcn_sched_barrier(0);
      }
      m_run = m_new;
    }
  };
  const bool_c<true> Y;
  const bool_c<false> N;

  // prologue: scores of tile 0
  wait_dma_newer(min(n_tiles - 1, PBUF - 2));
  barrier();
  phase_a(Y, N, N, ring[0], ring[0]);
  rescale(n_full > 0 ? phase_b(N, Y, N, ring[0], 0) : phase_b(N, Y, Y, ring[0], 0));
  // iteration t: scores of tile t + 1, weights and values of tile t
  auto iteration = [&](int t, auto masked) {
    // tile t + 1 landed for every wave; tile t - 1's slot is free
    wait_dma_newer(min(n_tiles - 2 - t, PBUF - 3));
    barrier();
    if (t + PBUF - 1 < n_tiles)
      tile_dma(src, (int64_t)(t + PBUF - 1) * STILE, n_blk, ring[(t + PBUF - 1) % PBUF], w, lane, off);
    const bf16_t* tc = ring[t % PBUF];
    const bf16_t* tn = ring[(t + 1) % PBUF];
    phase_a(Y, Y, Y, tn, tc);
    rescale(phase_b(Y, Y, masked, tc, (int64_t)(t + 1) * STILE));
  };
  // two loops, so that the masked body does not share registers with the
  // main one: tiles below n_full are whole for every row
  int t = 0;
  for (; t + 1 < n_tiles && t + 1 < n_full; ++t) iteration(t, N);
  for (; t + 1 < n_tiles; ++t) iteration(t, Y);
  {
    const bf16_t* tc = ring[(n_tiles - 1) % PBUF];
    phase_a(N, Y, Y, tc, tc);
    phase_b(Y, N, N, tc, 0);
  }

  if (!active) return;
  // oacc[ct][r] = O[query row r32][256 kh + 32 ct + 8 (r / 4) + 4 h32 + r % 4]
  const int head = hg * HB + (r32 & hmask);
  const float inv = 1.0f / l_run;
  TO* dst = o + ((int64_t)i_tok * H + head) * D_C + 256 * kh + 4 * h32;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = oacc[ct][4 * r4 + j] * inv;
      store4(dst + 32 * ct + 8 * r4, v);
    }
  if (lse != nullptr && h32 == 0 && kh == 0)
    lse[(int64_t)i_tok * H + head] = (m_run + __log2f(l_run)) * 0.69314718055994530942f;
}

template <typename TQ, typename TC, typename TO>
static void launch_pf_t(dim3 grid, hipStream_t st, const void* q, int64_t q_tok, int64_t cs,
                        int C, int H, int lhb, Seg reps, int64_t m, Seg raw, int64_t rb, float sl2, void* o,
                        float* lse) {
  hipLaunchKernelGGL((prefill_kernel_staged<TQ, TC, TO>), grid, dim3(NT), 0, st, (const TQ*)q, q_tok, cs,
                     C, H, lhb, reps, m, raw, rb, sl2, (TO*)o, lse);
}

template <typename TQ, typename TC>
static void launch_pf_o(int o_dtype, dim3 grid, hipStream_t st, const void* q, int64_t q_tok,
                        int64_t cs, int C, int H, int lhb, Seg reps, int64_t m, Seg raw, int64_t rb,
                        float sl2, void* o, float* lse) {
  if (o_dtype == LCA_BF16) launch_pf_t<TQ, TC, bf16_t>(grid, st, q, q_tok, cs, C, H, lhb, reps, m, raw, rb, sl2, o, lse);
  else launch_pf_t<TQ, TC, float>(grid, st, q, q_tok, cs, C, H, lhb, reps, m, raw, rb, sl2, o, lse);
}

static bool packed_rows_pf(const lca_latent_t& t) {
  return t.c != nullptr && t.dtype == LCA_BF16 &&
         static_cast<const char*>(t.kr) == static_cast<const char*>(t.c) + 2 * D_C &&
         t.kr_tok_stride == t.c_tok_stride;
}

template <typename TQ, class Src>
static void launch_pf2(int o_dtype, dim3 grid, hipStream_t st, const void* q, int64_t q_tok,
                       int64_t cs, int C, int H, int lhb, const Src& src, int64_t m, int64_t rb, float sl2,
                       void* o, float* lse) {
  if (o_dtype == LCA_BF16)
    hipLaunchKernelGGL((prefill_kernel<TQ, bf16_t, Src>), grid, dim3(256), 0, st, (const TQ*)q, q_tok, cs, C, H, lhb, src, m, rb, sl2, (bf16_t*)o, lse);
  else
    hipLaunchKernelGGL((prefill_kernel<TQ, float, Src>), grid, dim3(256), 0, st, (const TQ*)q, q_tok, cs, C, H, lhb, src, m, rb, sl2, (float*)o, lse);
}

// query tokens per workgroup and their log2 heads-per-block (64 query rows)
static void pf_rows(int H, int& lhb, int& n_tok) {
  const int hb = H < HB ? H : HB;
  lhb = 0;
  while ((1 << lhb) < hb) ++lhb;
  n_tok = 64 >> lhb;
}
// The fast kernel scales unscaled scores inside one fma before exp2, and
// masks with -inf; a scale of exactly 0 would turn -inf * 0 into NaN. The
// smallest normal float scale gives the same weights (every finite logit
// times it rounds to an exponent of 0, i.e. the uniform softmax that
// sm_scale = 0 means) and keeps -inf masked.
static float fast_scale(float sm_scale) {
  const float sl2 = sm_scale * 1.44269504088896340736f;
  return sl2 > 0.f ? sl2 : FLT_MIN;
}

hipError_t launch_prefill_paged(const void* q, int q_dtype, int64_t q_tok_stride, int64_t chunk_start,
                                int C, int H, const lca_latent_t& reps, int64_t m, const lca_paged_t& cache,
                                int seq, int64_t raw_begin, float sm_scale, void* o_latent, int o_dtype,
                                float* lse, hipStream_t stream) {
  int lhb, n_tok;
  pf_rows(H, lhb, n_tok);
  PagedDmaSrc src;
  src.rep = m > 0 ? static_cast<const char*>(reps.c) : nullptr;
  src.pages = static_cast<const char*>(cache.pages);
  src.table = cache.block_table + (int64_t)seq * cache.table_stride;
  src.tok = cache.row_stride * 2;
  src.m = m;
  src.raw_begin = raw_begin;
  src.P = cache.page_rows;
  const float sl2 = fast_scale(sm_scale);
  dim3 grid((unsigned)((C + n_tok - 1) / n_tok), (unsigned)head_blocks(H));
  if (q_dtype == LCA_BF16) launch_pf2<bf16_t>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, src, m, raw_begin, sl2, o_latent, lse);
  else launch_pf2<float>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, src, m, raw_begin, sl2, o_latent, lse);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* q, int q_dtype, int64_t q_tok_stride, int64_t chunk_start,
                          int C, int H, const lca_latent_t& reps, int64_t m,
                          const lca_latent_t& raw, int64_t raw_begin, float sm_scale,
                          void* o_latent, int o_dtype, float* lse, hipStream_t stream) {
  const float sl2 = sm_scale * 1.44269504088896340736f;
  int lhb, n_tok;
  pf_rows(H, lhb, n_tok);
  const bool fast = packed_rows_pf(raw) && (m == 0 || (packed_rows_pf(reps) && reps.c_tok_stride == raw.c_tok_stride)) &&
                    raw.c_tok_stride * 2 * STILE < ((int64_t)1 << 31);
  if (fast) {
    const float sl2_fast = fast_scale(sm_scale);
    DmaSrc src;
    src.rep = m > 0 ? static_cast<const char*>(reps.c) : nullptr;
    src.raw = static_cast<const char*>(raw.c) + raw_begin * raw.c_tok_stride * 2;
    src.tok = raw.c_tok_stride * 2;
    src.m = m;
    dim3 grid((unsigned)((C + n_tok - 1) / n_tok), (unsigned)head_blocks(H));
    if (q_dtype == LCA_BF16) launch_pf2<bf16_t>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, src, m, raw_begin, sl2_fast, o_latent, lse);
    else launch_pf2<float>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, src, m, raw_begin, sl2_fast, o_latent, lse);
    return hipGetLastError();
  }
  const Seg rs = to_seg(reps), ws = to_seg(raw);
  const int cdt = raw.dtype;
  dim3 grid((unsigned)((C + n_tok - 1) / n_tok), (unsigned)head_blocks(H));
  if (q_dtype == LCA_BF16) {
    if (cdt == LCA_BF16) launch_pf_o<bf16_t, bf16_t>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, rs, m, ws, raw_begin, sl2, o_latent, lse);
    else launch_pf_o<bf16_t, float>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, rs, m, ws, raw_begin, sl2, o_latent, lse);
  } else {
    if (cdt == LCA_BF16) launch_pf_o<float, bf16_t>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, rs, m, ws, raw_begin, sl2, o_latent, lse);
    else launch_pf_o<float, float>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, rs, m, ws, raw_begin, sl2, o_latent, lse);
  }
  return hipGetLastError();
}

}  // namespace lca
