// Entry tiles shared by the decode and prefill attention kernels.
//
// The attended set of a sequence is [representatives [0, m) ++ raw rows
// [raw_begin, ...)] (整体框架 of "Latent-Condensed Transformer for Efficient
// Long Context Modeling": representatives are concatenated with the window
// and attended with standard attention). A tile is 32 consecutive entries.
// The whole workgroup streams a tile from HBM with 16-byte loads (each thread
// keeps its 9 chunks of the next tile in registers while the current one is
// used; a wave instruction reads one row's 1 KB latent contiguously) and stores it row-major into LDS with a 16-byte pad per row, which
// keeps both the row-wise reads of the score product and the column-wise
// reads of the value product free of bank conflicts.
#pragma once
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int TILE = 32;                          // entries per tile
constexpr int LDS_ROW = D_ROW + 8;                // bf16 per LDS row (1168 bytes)
constexpr int NT = 256;                           // threads per workgroup
constexpr int CHUNKS = TILE * (D_ROW / 8);        // 16-byte chunks per tile (2304)
constexpr int CH_PER_T = CHUNKS / NT;             // 9
static_assert(CHUNKS % NT == 0, "tile chunks must split evenly over the workgroup");

template <typename TC>
struct EntrySrc {
  const TC* rc; const TC* rk; int64_t rc_tok, rk_tok;  // representatives of this sequence
  const TC* wc; const TC* wk; int64_t wc_tok, wk_tok;  // raw rows, entry m -> row raw_begin
  int64_t m;

  __device__ __forceinline__ void init(const Seg& reps, const Seg& raw, int b, int64_t m_,
                                       int64_t raw_begin) {
    rc = reps.c ? static_cast<const TC*>(reps.c) + (int64_t)b * reps.c_seq : nullptr;
    rk = reps.kr ? static_cast<const TC*>(reps.kr) + (int64_t)b * reps.kr_seq : nullptr;
    rc_tok = reps.c_tok; rk_tok = reps.kr_tok;
    wc = raw.c ? static_cast<const TC*>(raw.c) + (int64_t)b * raw.c_seq + raw_begin * raw.c_tok : nullptr;
    wk = raw.kr ? static_cast<const TC*>(raw.kr) + (int64_t)b * raw.kr_seq + raw_begin * raw.kr_tok : nullptr;
    wc_tok = raw.c_tok; wk_tok = raw.kr_tok;
    m = m_;
  }
  __device__ __forceinline__ const TC* c_row(int64_t e) const {
    return e < m ? rc + e * rc_tok : wc + (e - m) * wc_tok;
  }
  __device__ __forceinline__ const TC* k_row(int64_t e) const {
    return e < m ? rk + e * rk_tok : wk + (e - m) * wk_tok;
  }
};

// Global loads of entries [e0, e0 + TILE) (zeros past e_end). Thread t loads
// the 16-byte c_KV chunk (t % 64) of rows t/64 + 4i (one 1 KB row per wave
// instruction) and the k_R chunk (t % 8) of row t/8.
template <typename TC>
__device__ __forceinline__ void tile_load(const EntrySrc<TC>& src, int64_t e0, int64_t e_end,
                                          uint4 (&buf)[CH_PER_T], int tid) {
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t e = e0 + w + 4 * i;
    buf[i] = (e < e_end) ? load8_bf16(src.c_row(e) + 8 * lane) : make_uint4(0u, 0u, 0u, 0u);
  }
  const int64_t e = e0 + (tid >> 3);
  buf[8] = (e < e_end) ? load8_bf16(src.k_row(e) + 8 * (tid & 7)) : make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ void tile_store(bf16_t* lds, const uint4 (&buf)[CH_PER_T], int tid) {
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4*>(lds + (w + 4 * i) * LDS_ROW + 8 * lane) = buf[i];
  *reinterpret_cast<uint4*>(lds + (tid >> 3) * LDS_ROW + D_C + 8 * (tid & 7)) = buf[8];
}

// Entry (within a tile) that k slot kk of lane group kg stands for in the
// value product. It is the entry whose score the same lane holds after the
// transposed score product S^T = K Q^T (two 16-entry blocks, 4 rows each).
__device__ __forceinline__ int pv_entry(int kg, int kk) {
  return kk < 4 ? 4 * kg + kk : 16 + 4 * kg + (kk - 4);
}

// Value product from row fragments: R[kk] holds 8 consecutive latent columns
// (d = d0 + 8 col + 0..7) of tile entry pv_entry(kg, kk). Half-word shuffles
// turn them into the k-major operands of V^T, then
//   o[c] += V^T(d = d0 + 8 col + c) x P^T   for c = 0..7,
// where pb holds P[head col][pv_entry(kg, kk)] as 8 packed bf16. Afterwards
// o[c][r] accumulates O[head col][d0 + 32 kg + 8 r + c].
__device__ __forceinline__ void pv_from_rows(const uint4 (&R)[8], uint4 pb, f32x4_t* o) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    uint4 a;
    if (c & 1) {
      a.x = hi_pair(u4_get(R[0], w), u4_get(R[1], w));
      a.y = hi_pair(u4_get(R[2], w), u4_get(R[3], w));
      a.z = hi_pair(u4_get(R[4], w), u4_get(R[5], w));
      a.w = hi_pair(u4_get(R[6], w), u4_get(R[7], w));
    } else {
      a.x = lo_pair(u4_get(R[0], w), u4_get(R[1], w));
      a.y = lo_pair(u4_get(R[2], w), u4_get(R[3], w));
      a.z = lo_pair(u4_get(R[4], w), u4_get(R[5], w));
      a.w = lo_pair(u4_get(R[6], w), u4_get(R[7], w));
    }
    o[c] = mfma16x16x32(a, pb, o[c]);
  }
}

// 32-row variant: R[j] holds latent columns d0 + 8 (l%32) + 0..7 of the entry
// that k slot (l/32, j) stands for; o[c] += V^T(d = d0 + 8 (l%32) + c) x P^T
// with 32x32x16 MFMAs, pb holding P[query row l%32][slot entries].
__device__ __forceinline__ void pv_from_rows32(const uint4 (&R)[8], uint4 pb, f32x16_t* o) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    uint4 a;
    if (c & 1) {
      a.x = hi_pair(u4_get(R[0], w), u4_get(R[1], w));
      a.y = hi_pair(u4_get(R[2], w), u4_get(R[3], w));
      a.z = hi_pair(u4_get(R[4], w), u4_get(R[5], w));
      a.w = hi_pair(u4_get(R[6], w), u4_get(R[7], w));
    } else {
      a.x = lo_pair(u4_get(R[0], w), u4_get(R[1], w));
      a.y = lo_pair(u4_get(R[2], w), u4_get(R[3], w));
      a.z = lo_pair(u4_get(R[4], w), u4_get(R[5], w));
      a.w = lo_pair(u4_get(R[6], w), u4_get(R[7], w));
    }
    o[c] = mfma32x32x16(a, pb, o[c]);
  }
}

// Value product for one 128-column slab [d0, d0 + 128) of a padded row-major
// tile (LDS_ROW stride).
__device__ __forceinline__ void pv_slab(const bf16_t* tile, int d0, int kg, int col, uint4 pb,
                                        f32x4_t* o) {
  uint4 R[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    R[kk] = *reinterpret_cast<const uint4*>(tile + pv_entry(kg, kk) * LDS_ROW + d0 + 8 * col);
  pv_from_rows(R, pb, o);
}

// Online-softmax update for one tile. z[kk] are log2-domain logits of head
// `col` for entries pv_entry(kg, kk) (-inf when masked); the four lanes
// sharing a head (col, col+16, col+32, col+48) hold the tile's 32 entries.
// Returns the rescale factor for the running output and the packed P.
__device__ __forceinline__ float softmax_update(float (&z)[8], float& m_run, float& l_run,
                                                uint4& pb) {
  float tmax = z[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = fmaxf(m_run, tmax);
  float corr = 1.0f;
  float p[8];
  if (m_new == -INFINITY) {  // nothing visible yet
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = 0.f;
  } else {
    corr = exp2f(m_run - m_new);
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = exp2f(z[i] - m_new);
  }
  float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  ps += __shfl_xor(ps, 16);
  ps += __shfl_xor(ps, 32);
  l_run = l_run * corr + ps;
  m_run = m_new;
  pb = make_uint4(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]), pack_bf2(p[4], p[5]),
                  pack_bf2(p[6], p[7]));
  return corr;
}

// Online softmax with a lazy reference point: the running max m_run (log2
// domain) only moves when a logit exceeds it by more than LAZY_LOG2, and only
// then are the running sum and the accumulators o rescaled. In between, p =
// 2^(z - m_run) <= 2^LAZY_LOG2, which bf16 and fp32 hold easily; the final
// normalisation by l_run is exact either way. The test is uniform across a
// head's lanes, and skipping the rescale saves the 32 multiplies of o per tile.
constexpr float LAZY_LOG2 = 8.0f;
__device__ __forceinline__ void softmax_update_lazy(float (&z)[8], float& m_run, float& l_run,
                                                    uint4& pb, f32x4_t* o) {
  float tmax = z[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  if (__builtin_amdgcn_ballot_w64(tmax > m_run + LAZY_LOG2) != 0) {  // some head moves
    const float m_new = fmaxf(m_run, tmax);
    const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= corr;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] *= corr;
    m_run = m_new;
  }
  const float m_ref = m_run == -INFINITY ? 0.f : m_run;  // nothing visible yet: p = 0
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(z[i] - m_ref);
  float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  ps += __shfl_xor(ps, 16);
  ps += __shfl_xor(ps, 32);
  l_run += ps;
  pb = make_uint4(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]), pack_bf2(p[4], p[5]),
                  pack_bf2(p[6], p[7]));
}

}  // namespace lca
