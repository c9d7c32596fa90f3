// Chunked prefill attention over a condensed latent cache, gfx950.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// 整体框架: each query attends to the representatives of the groups older
// than its window plus the uncompressed rows (causal within the window). The
// groups a chunk sees are fixed before the chunk starts, so one chunk is a
// causal flash-attention over [reps ++ raw rows] shared by all H heads.
//
// In both kernels a wavefront holds 16 query rows (the 16 heads of one
// token; heads fill the 16-column side of every 16x16 MFMA tile, since all
// heads share the same keys and values). Entry tiles of 32 rows stream
// through LDS once per workgroup; per tile a wave forms S^T = K Q^T over the
// full 576 columns (18 MFMA 16x16x32 per 16 entries, its queries in
// registers), runs the online softmax in registers (four lanes per row) and
// accumulates O for all 512 latent columns (32 MFMA 16x16x32 per tile).
// Workgroups are issued heaviest (latest tokens) first.
//  prefill_kernel         packed bf16 rows: direct loads into a 4-slot ring,
//                         8 wavefronts (two per SIMD) per workgroup, one
//                         query block per workgroup.
//  prefill_sched_kernel   the same block function in persistent workgroups
//                         that take blocks from a counter in caller memory.
//  prefill_kernel_staged  any strides / f32 rows: register-staged tiles,
//                         4 wavefronts per workgroup.
#include <cfloat>

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

// prefill_kernel: the fast path for packed bf16 rows. Workgroup = 8
// wavefronts, two per SIMD; wave w holds 16 query rows (one token x 16
// heads; with Hb < 16 heads per key-value group, 16 / Hb tokens x Hb heads),
// the heads filling the 16-column side of every 16x16x32 MFMA, so a wave needs
// no partner: per 32-entry tile it forms S^T = K Q^T over all 576 columns (36
// MFMA, its queries in registers), runs the online softmax in registers (four
// lanes per query row) and accumulates O^T += V^T P^T over all 512 latent
// columns (32 MFMA; P straight from the score registers, V^T from transposed
// LDS reads). Its 72 (queries) + 128 (accumulators) + ~56 registers stay
// within the 256 that a second wave on every SIMD allows, and that second
// wave is what keeps the matrix cores fed while the other runs its softmax. Tiles stream HBM -> LDS by direct loads into a 4-slot
// ring (waves 0-3 issue them); one barrier per tile. Waves 0-3 run each tile
// as scores, softmax, values; waves 4-7 run the values of the previous tile
// first, so the two waves of a SIMD reach their softmax at different times.
constexpr int PFW = 8;     // wavefronts per workgroup
constexpr int PFRING = 4;  // ring depth: tiles t - 1 (values of waves 4-7), t, t + 1, t + 2
constexpr int PFKA = 2;    // score-product operands read this many products ahead
constexpr int PFVA = 3;    // value-product operands read this many products ahead

// max / sum over the four lanes holding one query row (lanes c, c + 16, c + 32, c + 48)
__device__ __forceinline__ float rows4_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One query block (128 query rows: 128 / Hb tokens x Hb heads of head group
// hg) of a chunk, by the whole workgroup.
template <typename TQ, typename TO, class Src>
__device__ __forceinline__ void prefill_block(
    bf16_t (&ring)[PFRING][STILE_ELEMS], const TQ* __restrict__ q, int64_t q_tok, int64_t chunk_start, int C,
    int H, int lhb, const Src& src, int64_t m, int64_t raw_begin, float scale_log2, TO* __restrict__ o,
    float* __restrict__ lse, int blk, int hg) {
  // an opaque copy of the thread index: in the persistent kernel nothing
  // derived from it is hoisted out of the block loop (there is no register
  // to hold it there)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = w < SNW;  // fills the tiles; runs each tile as scores, softmax, values
  const int kg = lane >> 4, col = lane & 15;
  // query row R = 16 w + col of the workgroup is (token R >> lhb, head
  // R % Hb), Hb = 2^lhb = min(H, 16): 128 / Hb tokens per workgroup
  const int n_tok = 128 >> lhb, hmask = (1 << lhb) - 1;
  const int tok0 = blk * n_tok;
  const int i_tok = tok0 + ((16 * w + col) >> lhb);
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
    slot_rowcol(w & (SNW - 1), i, lane, row, col16);
    off[i] = (uint32_t)(row * src.tok) + 16u * col16;
  }
  if (lead) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (t < n_tiles) tile_dma(src, (int64_t)t * STILE, n_blk, ring[t], w, lane, off);
  }

  // Q^T operand, k-step ks: query row col, columns 32 ks + 8 kg .. + 7
  const TQ* qh = q + (int64_t)i_ld * q_tok + (int64_t)(hg * HB + (col & hmask)) * D_ROW + 8 * kg;
  uint4 qa[18];
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) qa[ks] = load8_bf16(qh + 32 * ks);
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) retire(qa[ks]);

  // K operand of score product j (entry block eb = j % 2, k-step ks = j / 2):
  // lane (kg, col) reads row 16 eb + col, chunk 4 ks + kg, at
  // kb[ks & 1] + 64 (ks >> 1) + 16 eb rows (swz only flips the low three
  // chunk bits, and rows col and 16 + col share it).
  const int swc = swz(col);
  const int kb[2] = {8 * (col * (D_ROW / 8) + (kg ^ swc)), 8 * (col * (D_ROW / 8) + ((4 + kg) ^ swc))};
  auto kfrag = [&](const bf16_t* tile, int j) {
    const int ks = j >> 1, eb = j & 1;
    return *reinterpret_cast<const uint4*>(tile + kb[ks & 1] + 64 * (ks >> 1) + eb * 16 * D_ROW);
  };
  // V^T operand of value product ct (latent columns 16 ct .. + 15): lane (kg,
  // col) gets rows 4 kg .. + 3 (low half) and 16 + 4 kg .. + 3 (high half) of
  // column 16 ct + col, which pairs with the scores that lane holds; the 16
  // lanes of row group kg point at rows 4 kg + col / 4, columns
  // 16 ct + 4 (col % 4) .. + 3: vb[ct & 3] + 64 (ct >> 2).
  const int vr = 4 * kg + (col >> 2), swv = swz(vr);
  int vb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vb[j] = 8 * (vr * (D_ROW / 8) + ((2 * j + ((col >> 1) & 1)) ^ swv)) + 4 * (col & 1);
  auto vfrag = [&](const bf16_t* tile, int ct) {
    const bf16_t* pa = tile + vb[ct & 3] + 64 * (ct >> 2);
    const uint2 lo = lds_read_tr4(pa);
    const uint2 hi = lds_read_tr4(pa + 16 * D_ROW);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };

  f32x4_t oacc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) oacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane's share of the row sum

  // scores of tile t (entries 32 t + 16 eb + 4 kg + r in z[4 eb + r], unscaled,
  // -inf where causally hidden); returns the row max in scaled log2 units
  auto scores = [&](const bf16_t* tile, int t, float (&z)[8]) -> float {
    f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
    uint4 kf[PFKA + 1];
#pragma unroll
    for (int j = 0; j < PFKA; ++j) kf[j] = kfrag(tile, j);
#pragma unroll
    for (int j = 0; j < 36; ++j) {
      if (j + PFKA < 36) kf[(j + PFKA) % (PFKA + 1)] = kfrag(tile, j + PFKA);
      if (j & 1) s1 = mfma16x16x32(kf[j % (PFKA + 1)], qa[j >> 1], s1);
      else s0 = mfma16x16x32(kf[j % (PFKA + 1)], qa[j >> 1], s0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) { z[r] = s0[r]; z[4 + r] = s1[r]; }
    if (t >= n_full) {
      const int64_t e0 = (int64_t)t * STILE + 4 * kg;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (e0 + 16 * (i >> 2) + (i & 3) >= n_mine) z[i] = -INFINITY;
    }
    float tmax = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
    return rows4_max(tmax) * scale_log2;  // scale > 0, so the max commutes with it
  };
  // Lazy rescale (the reference max moves only when a row's max exceeds it
  // by more than 2^LAZY_LOG2; always on the first tile), then the weights p =
  // 2^(scale z - m_run) as bf16 and this lane's share of their sum.
  auto softmax = [&](const float (&z)[8], float tmax, uint4& pb) {
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + LAZY_LOG2) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        oacc[c] *= corr;
        __builtin_amdgcn_sched_barrier(0);
      }
      m_run = m_new;
    }
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(z[i], scale_log2, -m_ref));
    l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    pb = make_uint4(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]), pack_bf2(p[4], p[5]), pack_bf2(p[6], p[7]));
  };
  auto values = [&](const bf16_t* tile, const uint4& pb) {
    uint4 vf[PFVA + 1];
#pragma unroll
    for (int j = 0; j < PFVA; ++j) vf[j] = vfrag(tile, j);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
      if (ct + PFVA < 32) vf[(ct + PFVA) % (PFVA + 1)] = vfrag(tile, ct + PFVA);
      oacc[ct] = mfma16x16x32(vf[ct % (PFVA + 1)], pb, oacc[ct]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // top of iteration t: tile t has landed for every wave and every wave is
  // done with tile t - 2, whose slot takes tile t + 2
  auto top = [&](int t) {
    if (lead) wait_dma_newer(min(n_tiles - 1 - t, 1));
    barrier();
    if (lead && t + 2 < n_tiles)
      tile_dma(src, (int64_t)(t + 2) * STILE, n_blk, ring[(t + 2) % PFRING], w, lane, off);
  };

  float z[8];
  uint4 pb;
  if (lead) {
    for (int t = 0; t < n_tiles; ++t) {
      top(t);
      const bf16_t* tile = ring[t % PFRING];
      const float tmax = scores(tile, t, z);
      softmax(z, tmax, pb);
      values(tile, pb);
    }
  } else {
    for (int t = 0; t < n_tiles; ++t) {
      top(t);
      if (t > 0) values(ring[(t - 1) % PFRING], pb);
      const float tmax = scores(ring[t % PFRING], t, z);
      softmax(z, tmax, pb);
    }
    values(ring[(n_tiles - 1) % PFRING], pb);
  }

  const float l_row = rows4_sum(l_run);
  if (!active) return;
  // oacc[ct][r] = O[query row col][16 ct + 4 kg + r]
  const int head = hg * HB + (col & hmask);
  const float inv = 1.0f / l_row;
  TO* dst = o + ((int64_t)i_tok * H + head) * D_C + 4 * kg;
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) {
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = oacc[ct][r] * inv;
    store4(dst + 16 * ct, v);
  }
  if (lse != nullptr && kg == 0)
    lse[(int64_t)i_tok * H + head] = (m_run + __log2f(l_row)) * 0.69314718055994530942f;
}

template <typename TQ, typename TO, class Src>
__global__ __launch_bounds__(64 * PFW) void prefill_kernel(
    const TQ* __restrict__ q, int64_t q_tok, int64_t chunk_start, int C, int H, int lhb, Src src,
    int64_t m, int64_t raw_begin, float scale_log2, TO* __restrict__ o, float* __restrict__ lse) {
  __shared__ __align__(16) bf16_t ring[PFRING][STILE_ELEMS];
  // heavy workgroups (latest tokens) first
  prefill_block<TQ, TO, Src>(ring, q, q_tok, chunk_start, C, H, lhb, src, m, raw_begin, scale_log2, o, lse,
                             (int)gridDim.x - 1 - (int)blockIdx.x, blockIdx.y);
}

// The same blocks taken by persistent workgroups from a counter in global
// memory, heaviest first: workgroups are dealt to the XCDs round robin by
// index, so with one workgroup per block the hardware balances load only
// inside each XCD, and a slower XCD ends the chunk late; from the counter,
// a workgroup that finishes early takes the next block wherever it runs. A
// block's result does not depend on which workgroup computes it. sched[0]
// is the next block, sched[1] counts workgroups that found none left; the
// last of them puts both back to zero, so every launch starts and ends with
// a zeroed pair (the caller zeroes it once).
constexpr int PF_SCHED_WG = 256;  // persistent workgroups: one per CU of the part

template <typename TQ, typename TO, class Src>
__global__ __launch_bounds__(64 * PFW) void prefill_sched_kernel(
    const TQ* __restrict__ q, int64_t q_tok, int64_t chunk_start, int C, int H, int lhb, Src src,
    int64_t m, int64_t raw_begin, float scale_log2, TO* __restrict__ o, float* __restrict__ lse,
    int n_blocks, int n_hg, int* __restrict__ sched) {
  __shared__ __align__(16) bf16_t ring[PFRING][STILE_ELEMS];
  __shared__ int next;
  const int n_items = n_blocks * n_hg;
  for (;;) {
    // one barrier per block: the previous block's tile loop had barriers
    // after every wave read `next`, and its last tile is read by every
    // wave before the barrier here releases the ring
    if (threadIdx.x == 0) next = atomicAdd(sched, 1);
    __syncthreads();
    const int item = next;
    if (item < 0 || item >= n_items) break;  // (negative only if sched was not zeroed)
    prefill_block<TQ, TO, Src>(ring, q, q_tok, chunk_start, C, H, lhb, src, m, raw_begin, scale_log2, o, lse,
                               n_blocks - 1 - item / n_hg, item % n_hg);
  }
  if (threadIdx.x == 0 && atomicAdd(sched + 1, 1) == (int)(gridDim.x * gridDim.y) - 1) {
    atomicExch(sched, 0);
    atomicExch(sched + 1, 0);
  }
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
                       void* o, float* lse, int* sched = nullptr) {
  grid.x = (unsigned)((C + (128 >> lhb) - 1) / (128 >> lhb));  // 128 query rows per workgroup
  if (sched != nullptr) {
    // one resident workgroup per CU (the ring fills its LDS), at most one per block
    const int items = (int)(grid.x * grid.y);
    const dim3 gs((unsigned)(items < PF_SCHED_WG ? items : PF_SCHED_WG));
    if (o_dtype == LCA_BF16)
      hipLaunchKernelGGL((prefill_sched_kernel<TQ, bf16_t, Src>), gs, dim3(64 * PFW), 0, st, (const TQ*)q, q_tok, cs, C, H, lhb, src, m, rb, sl2, (bf16_t*)o, lse, (int)grid.x, (int)grid.y, sched);
    else
      hipLaunchKernelGGL((prefill_sched_kernel<TQ, float, Src>), gs, dim3(64 * PFW), 0, st, (const TQ*)q, q_tok, cs, C, H, lhb, src, m, rb, sl2, (float*)o, lse, (int)grid.x, (int)grid.y, sched);
    return;
  }
  if (o_dtype == LCA_BF16)
    hipLaunchKernelGGL((prefill_kernel<TQ, bf16_t, Src>), grid, dim3(64 * PFW), 0, st, (const TQ*)q, q_tok, cs, C, H, lhb, src, m, rb, sl2, (bf16_t*)o, lse);
  else
    hipLaunchKernelGGL((prefill_kernel<TQ, float, Src>), grid, dim3(64 * PFW), 0, st, (const TQ*)q, q_tok, cs, C, H, lhb, src, m, rb, sl2, (float*)o, lse);
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
                                float* lse, hipStream_t stream, int* sched) {
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
  if (q_dtype == LCA_BF16) launch_pf2<bf16_t>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, src, m, raw_begin, sl2, o_latent, lse, sched);
  else launch_pf2<float>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, src, m, raw_begin, sl2, o_latent, lse, sched);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* q, int q_dtype, int64_t q_tok_stride, int64_t chunk_start,
                          int C, int H, const lca_latent_t& reps, int64_t m,
                          const lca_latent_t& raw, int64_t raw_begin, float sm_scale,
                          void* o_latent, int o_dtype, float* lse, hipStream_t stream, int* sched) {
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
    if (q_dtype == LCA_BF16) launch_pf2<bf16_t>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, src, m, raw_begin, sl2_fast, o_latent, lse, sched);
    else launch_pf2<float>(o_dtype, grid, stream, q, q_tok_stride, chunk_start, C, H, lhb, src, m, raw_begin, sl2_fast, o_latent, lse, sched);
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
