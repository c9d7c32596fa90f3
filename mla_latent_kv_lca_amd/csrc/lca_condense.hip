// LCA condensation kernels for gfx950.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// 关键设计 1 (summary query = mean of the most recent g queries, per-token
// importance, softmax weights, weighted pooling of c_KV) and 关键设计 2 (the
// group's k_R is the k_R of its most important token).
//
// Kernels:
//  qbar_kernel      one workgroup per summary query: mean over g query tokens
//                   and H heads of 576-wide absorbed queries -> fp32 workspace.
//  qbar_part_kernel / qbar_final_kernel: the same mean for one summary query
//                   per sequence, in 8 part sums over 8 workgroups, then added.
//  condense_kernel  one wavefront per group. Lane l owns latent columns
//                   [8l, 8l+8) and RoPE column l of all g rows, so each row
//                   load is one fully coalesced 1 KB (c_KV) + 128 B (k_R)
//                   wave access and every row's score is formed by the same
//                   sequence of operations (identical rows give bitwise equal
//                   scores). The g partial dot products are reduced across
//                   the 64 lanes with a halving butterfly (g/2 + g/4 + ...
//                   exchanges instead of 6 g), all exchanges stay in
//                   registers (lane-half swaps and DPP), the anchor is the
//                   lowest lane of a ballot at the group max, the weights
//                   reach every lane as scalars, and the pooled row is
//                   accumulated in fp32.
// The work is HBM streaming (about 2 flop per byte): no matrix cores.
#include <algorithm>

#include "lca_device.h"
#include "lca_internal.h"
#include "lca_stream.h"
#include "lca_up_rows.h"

namespace lca {

// ---------------------------------------------------------------- K0 -------
constexpr int QBAR_PH = 14;                  // row phases
constexpr int QBAR_THREADS = 72 * QBAR_PH;   // 72 column chunks of 8 x 14 row phases

// Per-group summary queries: one workgroup per summary query; thread (chunk
// c, phase p) sums rows p, p + 14, ... of the g*H query rows, eight loads in
// flight at a time; the 14 phase partials are then added in phase order.
template <typename TQ>
__global__ __launch_bounds__(QBAR_THREADS) void qbar_kernel(
    const TQ* __restrict__ q, int64_t q_seq, int64_t q_tok, int H, int g, int64_t row0,
    int64_t step, int n_q, float* __restrict__ qbar) {
  const int jq = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, ch = t % 72, ph = t / 72;
  const TQ* base = q + (int64_t)b * q_seq + (row0 + (int64_t)jq * step) * q_tok + ch * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int rows = g * H;
  for (int r0 = ph; r0 < rows; r0 += 8 * QBAR_PH) {
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * QBAR_PH;
      if (r < rows) {
        const int tok = r / H, h = r - tok * H;
        load8_f32(base + (int64_t)tok * q_tok + h * D_ROW, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[u][i];
  }
  __shared__ float sh[QBAR_PH][D_ROW];
#pragma unroll
  for (int i = 0; i < 8; ++i) sh[ph][ch * 8 + i] = acc[i];
  __syncthreads();
  const float inv = 1.0f / (float)rows;
  for (int c = t; c < D_ROW; c += QBAR_THREADS) {
    float s = sh[0][c];
    for (int p = 1; p < QBAR_PH; ++p) s += sh[p][c];
    qbar[((int64_t)b * n_q + jq) * D_ROW + c] = s * inv;
  }
}

// One summary query per sequence (decode): its g*H rows are cut into
// QBAR_PARTS contiguous parts summed by separate workgroups (so a handful of
// sequences still spread over many CUs), then qbar_final_kernel adds the part
// sums in part order. Part workgroup: thread (chunk c, phase p) sums rows
// p, p + 4, ... of its part, all its loads in flight at once, and the four
// phase sums are added in phase order.
constexpr int QP_PH = 4;
constexpr int QP_THREADS = 72 * QP_PH;
template <typename TQ>
__global__ __launch_bounds__(QP_THREADS) void qbar_part_kernel(
    const TQ* __restrict__ q, int64_t q_seq, int64_t q_tok, int H, int g, int64_t row0,
    float* __restrict__ part) {
  const int p = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, ch = t % 72, ph = t / 72;
  const int rows = g * H, per = (rows + QBAR_PARTS - 1) / QBAR_PARTS;
  const int r_begin = p * per, r_end = min(rows, r_begin + per);
  const TQ* base = q + (int64_t)b * q_seq + row0 * q_tok + ch * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r0 = r_begin + ph; r0 < r_end; r0 += 8 * QP_PH) {
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * QP_PH;
      if (r < r_end) {
        const int tok = r / H, h = r - tok * H;
        load8_f32(base + (int64_t)tok * q_tok + h * D_ROW, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[u][i];
  }
  __shared__ float sh[QP_PH][D_ROW];
#pragma unroll
  for (int i = 0; i < 8; ++i) sh[ph][ch * 8 + i] = acc[i];
  __syncthreads();
  for (int c = t; c < D_ROW; c += QP_THREADS) {
    float s = sh[0][c];
    for (int k = 1; k < QP_PH; ++k) s += sh[k][c];
    part[((int64_t)b * QBAR_PARTS + p) * D_ROW + c] = s;
  }
}
// Column c of the summary query from the part sums (pp = part sums of the
// sequence + c): added in part order, then scaled. The streaming condense
// kernel forms its summary query with this same function, so both paths
// hold bitwise equal values.
__device__ __forceinline__ float qbar_from_parts(const float* pp, int rows) {
  float s = pp[0];
#pragma unroll
  for (int k = 1; k < QBAR_PARTS; ++k) s += pp[k * D_ROW];
  return s * (1.0f / (float)rows);
}

__global__ __launch_bounds__(D_ROW) void qbar_final_kernel(const float* __restrict__ part, int rows,
                                                           float* __restrict__ qbar) {
  const int b = blockIdx.x, c = threadIdx.x;
  qbar[(int64_t)b * D_ROW + c] = qbar_from_parts(part + (int64_t)b * QBAR_PARTS * D_ROW + c, rows);
}

// ---------------------------------------------------------------- K1 -------
// v_cndmask with the lane mask in an SGPR pair, kept opaque: written as a C
// select, the compiler turns "upper ? v[i] : v[i + half]" into a variable
// index into v, which it then expands into a compare-and-select per element.
__device__ __forceinline__ float lane_select(uint64_t take_b, float a, float b) {
  float r;
  asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(take_b));
  return r;
}

// Cross-lane exchanges of the group reductions, all in registers. Lane bits
// 5 and 4: v_permlane32_swap / v_permlane16_swap swap register halves in one
// instruction. Bit 3: DPP rotate of each 16-lane row by 8 (lane xor 8).
// Bit 2: DPP half-row mirror (lane l <-> 7 - l within each 8 lanes, which
// pairs every lane that has bit 2 clear with one that has it set). Bits 1
// and 0: DPP quad permutations (lane xor 2, lane xor 1). Every pairing is an
// involution, so both lanes of a pair combine the same two values.
template <int MASK>
__device__ __forceinline__ float dpp_partner(float v) {
  static_assert(MASK == 8 || MASK == 4 || MASK == 2 || MASK == 1, "DPP exchange");
  constexpr int ctrl = MASK == 8 ? 0x128 : MASK == 4 ? 0x141 : MASK == 2 ? 0x4e : 0xb1;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, false));
}
// lanes whose bit MASK is set
template <int MASK>
constexpr uint64_t lanes_with_bit() {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l)
    if (l & MASK) m |= uint64_t(1) << l;
  return m;
}

// Sum (or max) of v over the two lanes of a pair differing in bit MASK.
template <int MASK, bool MAX>
__device__ __forceinline__ float pair_op(float v) {
  float a, b;
  if constexpr (MASK == 32 || MASK == 16) {
    const auto r = MASK == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                              : __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    a = v;
    b = dpp_partner<MASK>(v);
  }
  return MAX ? fmaxf(a, b) : a + b;
}
// Fold v over lane bits MASK, MASK / 2, ..., STOP (MASK >= STOP, powers of 2).
template <int MASK, int STOP, bool MAX>
__device__ __forceinline__ float fold_lanes(float v) {
  if constexpr (MASK >= STOP && MASK >= 1) return fold_lanes<MASK / 2, STOP, MAX>(pair_op<MASK, MAX>(v));
  else return v;
}

// One halving step on lane bit MASK: the lanes with the bit clear end with
// lo summed over the pair, the lanes with it set with hi.
template <int MASK>
__device__ __forceinline__ float halve(float lo, float hi) {
  if constexpr (MASK == 32 || MASK == 16) {
    // lanes below the half boundary get (lo, lo of the partner), the others
    // (hi of the partner, hi)
    const auto r = MASK == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false)
                              : __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    constexpr uint64_t upper = lanes_with_bit<MASK>();
    const float send = lane_select(upper, hi, lo);  // lanes with the bit set send lo
    const float keep = lane_select(upper, lo, hi);
    return keep + dpp_partner<MASK>(send);
  }
}
template <int LG, int ST>
__device__ __forceinline__ void halving_stages(float (&v)[1 << LG]) {
  if constexpr (ST < LG) {
    constexpr int MASK = 32 >> ST, HALF = (1 << LG) >> (ST + 1);
#pragma unroll
    for (int i = 0; i < HALF; ++i) v[i] = halve<MASK>(v[i], v[i + HALF]);
    halving_stages<LG, ST + 1>(v);
  }
}

// Reduce v[0..G) over all 64 lanes; afterwards every lane holds the total of
// row (lane >> (6 - LG)), bitwise the same in all lanes of the row, and every
// row's total is formed by the same tree of additions.
template <int LG>
__device__ __forceinline__ float reduce_rows(float (&v)[1 << LG]) {
  halving_stages<LG, 0>(v);
  return fold_lanes<(32 >> LG), 1, false>(v[0]);
}

// Group rows are read exactly once: non-temporal (streaming) loads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
template <typename TC> struct RowChunk;  // 8 latent elements of one row held by a lane
template <> struct RowChunk<bf16_t> {
  uint4 v;
  __device__ void load(const bf16_t* p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    v = make_uint4(t.x, t.y, t.z, t.w);
  }
  __device__ float get(int i) const {
    const uint32_t w = u4_get(v, i >> 1);
    return (i & 1) ? bf_hi(w) : bf_lo(w);
  }
};
template <> struct RowChunk<float> {
  float v[8];
  __device__ void load(const float* p) {
    const f32x4v_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p));
    const f32x4v_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p) + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ float get(int i) const { return v[i]; }
};

// Scores, weights and representative of one group held by a wavefront (lane
// owns latent columns 8 lane .. 8 lane + 7 and RoPE column lane of every row).
// mode (wave-uniform): LCA_MODE_LCA pools the latents and takes the anchor's
// RoPE key; LCA_MODE_POOL_ROPE pools the RoPE keys too; LCA_MODE_ANCHOR
// keeps the anchor's row (the ablation variants of 消融实验).
template <typename TC, int LG>
struct GroupResult {
  float acc[8];   // representative latent columns of this lane
  int arg;        // anchor row within the group (wave-uniform)
  float a_mine;   // weight of row my_row
  int my_row;
  float kval;     // representative RoPE column of this lane
};
template <typename TC, int LG>
__device__ __forceinline__ GroupResult<TC, LG> condense_group(const RowChunk<TC> (&rows)[1 << LG],
                                                             const TC (&krv)[1 << LG], const float (&qc)[8],
                                                             float qr, float sm_scale, int lane, int mode) {
  constexpr int G = 1 << LG, SH = 6 - LG;  // a row's total sits in lanes [r << SH, (r + 1) << SH)
  GroupResult<TC, LG> out;
  // partial scores of this lane's columns, same operation order for every row
  float s[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    float a = rows[r].get(0) * qc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) a = fmaf(rows[r].get(i), qc[i], a);
    s[r] = fmaf(to_f32(krv[r]), qr, a);
  }
  const float score = reduce_rows<LG>(s);
  out.my_row = lane >> SH;
  // group max over the row bits; the anchor is the first row that attains it
  const float mx = fold_lanes<32, (64 >> LG), true>(score);
  const uint64_t at_max = __builtin_amdgcn_ballot_w64(score == mx);
  out.arg = at_max ? (int)(__builtin_ctzll(at_max) >> SH) : 0;
  const float e = __expf(sm_scale * (score - mx));
  const float tot = fold_lanes<32, (64 >> LG), false>(e);
  out.a_mine = e / tot;
  // alpha_r read from the first lane of row r (wave-uniform, so it lives in
  // a scalar register)
  float al[G];
#pragma unroll
  for (int r = 0; r < G; ++r)
    al[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(out.a_mine), r << SH));
  // the anchor's own row (arg is uniform: a scalar branch per row)
  int ka = 0;
#pragma unroll
  for (int r = 1; r < G; ++r)
    if (r == out.arg) ka = r;
  if (mode == LCA_MODE_ANCHOR) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out.acc[i] = rows[0].get(i);
#pragma unroll
    for (int r = 1; r < G; ++r)
      if (r == ka) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out.acc[i] = rows[r].get(i);
      }
  } else {
    // pooled latent: sum_r alpha_r c_r in row order
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) out.acc[i] = (r == 0) ? al[r] * rows[r].get(i) : fmaf(al[r], rows[r].get(i), out.acc[i]);
  }
  if (mode == LCA_MODE_POOL_ROPE) {
    out.kval = al[0] * to_f32(krv[0]);
#pragma unroll
    for (int r = 1; r < G; ++r) out.kval = fmaf(al[r], to_f32(krv[r]), out.kval);
  } else {
    out.kval = to_f32(krv[0]);
#pragma unroll
    for (int r = 1; r < G; ++r)
      if (r == ka) out.kval = to_f32(krv[r]);
  }
  return out;
}

template <typename TC, typename TR, int LG>
__global__ __launch_bounds__(256) void condense_kernel(
    const TC* __restrict__ c, const TC* __restrict__ kr, int64_t c_seq, int64_t c_tok,
    int64_t kr_seq, int64_t kr_tok, const float* __restrict__ qbar, int per_group_q,
    int64_t n_q, int64_t group_begin, int64_t n_groups, float sm_scale, TR* __restrict__ rc,
    TR* __restrict__ rk, int64_t rc_seq, int64_t rc_tok, int64_t rk_seq, int64_t rk_tok,
    int32_t* __restrict__ anchor, int64_t anchor_seq, float* __restrict__ alpha,
    int64_t alpha_seq, int mode) {
  constexpr int G = 1 << LG;
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_groups) return;  // wave-uniform
  const int b = blockIdx.y;
  const int64_t j = group_begin + n;

  const float* qb = qbar + ((int64_t)b * n_q + (per_group_q ? n : 0)) * D_ROW;
  float qc[8];
  load8_f32(qb + 8 * lane, qc);
  const float qr = qb[D_C + lane];

  const TC* cg = c + (int64_t)b * c_seq + j * G * c_tok + 8 * lane;
  const TC* kg = kr + (int64_t)b * kr_seq + j * G * kr_tok + lane;
  RowChunk<TC> rows[G];
  TC krv[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    rows[r].load(cg + r * c_tok);
    krv[r] = __builtin_nontemporal_load(kg + r * kr_tok);
  }
  const GroupResult<TC, LG> gr = condense_group<TC, LG>(rows, krv, qc, qr, sm_scale, lane, mode);
  store8(rc + (int64_t)b * rc_seq + j * rc_tok + 8 * lane, gr.acc);
  rk[(int64_t)b * rk_seq + j * rk_tok + lane] = from_f32<TR>(gr.kval);
  if (lane == 0) anchor[(int64_t)b * anchor_seq + j] = (int32_t)(j * G + gr.arg);
  if (alpha != nullptr && (lane & ((64 >> LG) - 1)) == 0)
    alpha[(int64_t)b * alpha_seq + j * G + gr.my_row] = gr.a_mine;
}

// ---------------------------------------------------------------- K1r ------
// Streaming variant for packed bf16 rows and one summary query per sequence
// (decode-time condensation), g = 8 or 16. The wavefronts of a sequence take
// its groups round robin (wave w of W: groups w, w + W, ...), so at any time
// the loads and the output writes of all waves fall in one narrow window of
// memory. Group tiles (g rows x 1,152 bytes) stream from HBM straight into a
// wave-private LDS ring by direct non-temporal loads, so the next groups are
// in flight while one is scored and pooled, and the workgroups stay resident
// instead of being re-dispatched per group. Outputs are written through to
// memory (device-scope stores): a steady trickle of writes costs the read
// stream less than bursts of write-backs from L2.
// The arithmetic per group is exactly that of condense_kernel (same operand
// order), so both kernels give bitwise equal results.
// Completion of a tile is tracked with vmcnt, which also counts this wave's
// stores: every group issues exactly NST stores (pooled row, anchor k_R,
// anchor index, and the weights when requested), after the loads of the tile
// that reuses its slot; the stores are written in asm so that their number
// is exact.
template <int LG>
struct RingCfg {
  static constexpr int G = 1 << LG;
  static constexpr int TILE = G * D_ROW;                      // bf16 elements per group tile
  static constexpr int NS = LG == 3 ? 4 : 2;                  // slots per wave
  static constexpr int NI = G * (D_ROW / 8) / 64;             // load instructions per tile
};
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// device-scope (write-through) vector stores, one instruction each
// (a VALU write to the data registers of a 16-byte store must wait one cycle)
__device__ __forceinline__ void st_wt16(void* p, uint4 v) {
  const u32x4_t d = {v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 0" ::"v"(p), "v"(d) : "memory");
}
__device__ __forceinline__ void st_wt4(void* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_wt2(void* p, uint32_t v) {
  asm volatile("global_store_short %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// Wait until the tile issued before `stores_after` groups' stores and
// `tiles_after` later tiles has landed (vmcnt counts loads and stores in
// issue order).
template <int LG, bool ALPHA>
__device__ __forceinline__ void wait_tile(int stores_after, int tiles_after) {
  constexpr int NI = RingCfg<LG>::NI, NS = RingCfg<LG>::NS, NST = ALPHA ? 4 : 3;
  // stores_after in [0, NS], tiles_after in [0, NS - 1]
  if constexpr (NS == 2) {
    switch (stores_after * 2 + tiles_after) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<NI>(); break;
      case 2: wait_vm<NST>(); break;
      case 3: wait_vm<NST + NI>(); break;
      case 4: wait_vm<2 * NST>(); break;
      default: wait_vm<2 * NST + NI>(); break;
    }
  } else {
    static_assert(NS == 4 && 4 * NST + 3 * NI <= 63, "vmcnt immediates");
    switch (stores_after * 4 + tiles_after) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<NI>(); break;
      case 2: wait_vm<2 * NI>(); break;
      case 3: wait_vm<3 * NI>(); break;
      case 4: wait_vm<NST>(); break;
      case 5: wait_vm<NST + NI>(); break;
      case 6: wait_vm<NST + 2 * NI>(); break;
      case 7: wait_vm<NST + 3 * NI>(); break;
      case 8: wait_vm<2 * NST>(); break;
      case 9: wait_vm<2 * NST + NI>(); break;
      case 10: wait_vm<2 * NST + 2 * NI>(); break;
      case 11: wait_vm<2 * NST + 3 * NI>(); break;
      case 12: wait_vm<3 * NST>(); break;
      case 13: wait_vm<3 * NST + NI>(); break;
      case 14: wait_vm<3 * NST + 2 * NI>(); break;
      case 15: wait_vm<3 * NST + 3 * NI>(); break;
      case 16: wait_vm<4 * NST>(); break;
      case 17: wait_vm<4 * NST + NI>(); break;
      case 18: wait_vm<4 * NST + 2 * NI>(); break;
      default: wait_vm<4 * NST + 3 * NI>(); break;
    }
  }
}

template <int LG, bool ALPHA>
__global__ __launch_bounds__(256) void condense_ring_kernel(
    const char* __restrict__ cache, int64_t seq_b, int64_t tok_b, const float* __restrict__ qpart,
    int q_rows, int64_t group_begin, int64_t n_groups, float sm_scale,
    bf16_t* __restrict__ rc, bf16_t* __restrict__ rk, int64_t rc_seq, int64_t rc_tok,
    int64_t rk_seq, int64_t rk_tok, int32_t* __restrict__ anchor, int64_t anchor_seq,
    float* __restrict__ alpha, int64_t alpha_seq) {
  using Cfg = RingCfg<LG>;
  constexpr int G = Cfg::G, NS = Cfg::NS, NI = Cfg::NI;
  __shared__ __align__(16) bf16_t ring[4][NS][Cfg::TILE];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  // this wave's groups: wg + k nw, k = 0 .. count - 1
  const int64_t wg = (int64_t)blockIdx.y * 4 + w, nw = (int64_t)gridDim.y * 4;
  const int64_t count = wg < n_groups ? (n_groups - 1 - wg) / nw + 1 : 0;
  if (count == 0) return;  // wave-uniform; the kernel has no barriers

  // the summary query straight from the part sums (no separate final pass)
  const float* qp = qpart + (int64_t)b * QBAR_PARTS * D_ROW;
  float qc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qc[i] = qbar_from_parts(qp + 8 * lane + i, q_rows);
  const float qr = qbar_from_parts(qp + D_C + lane, q_rows);
  // the compiler waits for these loads here, before any tile is in flight
  asm volatile("" ::"v"(qc[0]), "v"(qc[1]), "v"(qc[2]), "v"(qc[3]), "v"(qc[4]), "v"(qc[5]), "v"(qc[6]),
               "v"(qc[7]), "v"(qr));

  // tile load: LDS position P = 64 i + lane holds bytes [16 P, 16 P + 16) of
  // the group's rows laid end to end (row P / 72, chunk P % 72)
  uint32_t off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int P = 64 * i + lane, row = P / (D_ROW / 8), c16 = P - row * (D_ROW / 8);
    off[i] = (uint32_t)(row * tok_b) + 16u * c16;
  }
  const char* seq = cache + (int64_t)b * seq_b;
  auto issue = [&](int64_t k) {
    const char* g0 = seq + (group_begin + wg + k * nw) * G * tok_b;
    dma16_rows<1024u, true>(g0, off, lds_off(&ring[w][k % NS][0]));
  };
#pragma unroll
  for (int k = 0; k < NS; ++k)
    if (k < count) issue(k);

  for (int64_t k = 0; k < count; ++k) {
    // after tile k was issued: the stores of groups max(0, k - NS) .. k - 1
    // and the tiles k + 1 .. k + NS - 1
    wait_tile<LG, ALPHA>((int)min(k, (int64_t)NS), (int)min(count - 1 - k, (int64_t)NS - 1));
    const bf16_t* tile = &ring[w][k % NS][0];
    RowChunk<bf16_t> rows[G];
    bf16_t krv[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      rows[r].v = *reinterpret_cast<const uint4*>(tile + r * D_ROW + 8 * lane);
      krv[r] = tile[r * D_ROW + D_C + lane];
    }
    // the rows are in registers: the slot takes group k + NS right away
    if (k + NS < count) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(k + NS);
    }
    const int64_t j = group_begin + wg + k * nw;
    const GroupResult<bf16_t, LG> gr = condense_group<bf16_t, LG>(rows, krv, qc, qr, sm_scale, lane, LCA_MODE_LCA);
    // exactly NST vector stores per group (counted by wait_tile)
    st_wt16(rc + (int64_t)b * rc_seq + j * rc_tok + 8 * lane,
            make_uint4(pack_bf2(gr.acc[0], gr.acc[1]), pack_bf2(gr.acc[2], gr.acc[3]),
                       pack_bf2(gr.acc[4], gr.acc[5]), pack_bf2(gr.acc[6], gr.acc[7])));
    st_wt2(rk + (int64_t)b * rk_seq + j * rk_tok + lane, f2bf(gr.kval));
    if (lane == 0) st_wt4(anchor + (int64_t)b * anchor_seq + j, (uint32_t)(j * G + gr.arg));
    if (ALPHA && (lane & ((64 >> LG) - 1)) == 0)
      st_wt4(alpha + (int64_t)b * alpha_seq + j * G + gr.my_row, __float_as_uint(gr.a_mine));
  }
}

// ---------------------------------------------------------------- K1p ------
// Ragged batch over a paged cache (packed bf16 rows and representatives,
// one summary query per sequence): wavefront n of sequence b condenses group
// seq_group_begin[b] + n when n < seq_n_groups[b]. A group lies inside one
// page (page_rows is a multiple of g), found with one scalar table load.
template <int LG>
__global__ __launch_bounds__(256) void condense_paged_kernel(
    const bf16_t* __restrict__ pages, int64_t row_stride, int page_rows, const int32_t* __restrict__ table,
    int64_t table_stride, const int32_t* __restrict__ seq_group_begin, const int32_t* __restrict__ seq_n_groups,
    const float* __restrict__ qbar, int per_group_q, int64_t n_q, float sm_scale, bf16_t* __restrict__ rc,
    int64_t rc_seq, int64_t rc_tok,
    int32_t* __restrict__ anchor, int64_t anchor_seq, float* __restrict__ alpha, int64_t alpha_seq) {
  constexpr int G = 1 << LG;
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (n >= seq_n_groups[b]) return;  // wave-uniform
  const int64_t j = seq_group_begin[b] + n, t0 = j * G;
  const int64_t page = table[(int64_t)b * table_stride + t0 / page_rows];
  const bf16_t* rows0 = pages + (page * page_rows + t0 % page_rows) * row_stride;

  const float* qb = qbar + ((int64_t)b * n_q + (per_group_q ? n : 0)) * D_ROW;
  float qc[8];
  load8_f32(qb + 8 * lane, qc);
  const float qr = qb[D_C + lane];
  RowChunk<bf16_t> rows[G];
  bf16_t krv[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    rows[r].load(rows0 + r * row_stride + 8 * lane);
    krv[r] = __builtin_nontemporal_load(rows0 + r * row_stride + D_C + lane);
  }
  const GroupResult<bf16_t, LG> gr = condense_group<bf16_t, LG>(rows, krv, qc, qr, sm_scale, lane, LCA_MODE_LCA);
  bf16_t* dst = rc + (int64_t)b * rc_seq + j * rc_tok;
  store8(dst + 8 * lane, gr.acc);
  dst[D_C + lane] = (bf16_t)f2bf(gr.kval);
  if (lane == 0) anchor[(int64_t)b * anchor_seq + j] = (int32_t)(t0 + gr.arg);
  if (alpha != nullptr && (lane & ((64 >> LG) - 1)) == 0)
    alpha[(int64_t)b * alpha_seq + j * G + gr.my_row] = gr.a_mine;
}

// ---------------------------------------------------------------- step ----
// One decode step's incremental condensation and bookkeeping over a ragged
// batch on a paged cache, as one launch (so a decode step is a fixed
// sequence of launches). Workgroup b = sequence b, QS_THREADS threads:
//  - this step's query (token L = seq_raw_end[b]) goes to ring row L mod g;
//  - after the step's row is appended the cache holds L + 1 tokens; when
//    L + 1 - w >= (m + 1) g, group m is complete and is condensed (整体框架;
//    关键设计 1: the mean of the most recent g queries, i.e. of the g ring
//    rows, this step's query included, over all H heads) with the same group
//    function as the other condense kernels, by wave 0;
//  - the state for the next step is written: m, the raw range [m g, L + 1),
//    and the position and physical cache row of token L + 1.
// Every thread reads the state before the barrier that precedes its update.
// The summary query reads this step's query from q, never from the ring row
// the same workgroup writes.
constexpr int QS_THREADS = 256;            // threads of a step workgroup
constexpr int QS_PH = QS_THREADS / 72;      // row phases of the summary-query sum (3)
static_assert(QS_THREADS == 64 * UPR_WAVES, "step workgroups also run inside up_rows_kernel");

template <typename TQ, int LG>
struct CondenseStep {
  int B;  // sequences (step workgroups)
  const bf16_t* pages;
  int64_t row_stride;
  int page_rows;
  const int32_t* table;
  int64_t table_stride;
  int64_t w;
  const TQ* q;
  int64_t q_seq;
  int H;
  TQ* ring;
  int64_t ring_seq;
  float sm_scale;
  bf16_t* rc;
  int64_t rc_seq, rc_tok;
  int32_t* anchor;
  int64_t anchor_seq;
  int32_t* seq_m;
  int32_t* seq_raw_begin;
  int32_t* seq_raw_end;
  int32_t* pos;
  int64_t* dst_row;

  __device__ void run(int b) const {
    constexpr int G = 1 << LG;
    const int t = threadIdx.x, ch = t % 72, ph = t / 72;
    const int64_t L = seq_raw_end[b];
    const int64_t m = seq_m[b];
    const int cur = (int)(L & (G - 1));
    const bool cond = L + 1 - w >= (m + 1) * G;
    const int64_t row_elems = (int64_t)H * D_ROW;
    const TQ* qb = q + (int64_t)b * q_seq;
    TQ* rb = ring + (int64_t)b * ring_seq;

    // this step's query into its ring row (8 elements per store)
    for (int64_t i = t; i < row_elems / 8; i += QS_THREADS) {
      if constexpr (sizeof(TQ) == 2) {
        *reinterpret_cast<uint4*>(rb + cur * row_elems + 8 * i) = *reinterpret_cast<const uint4*>(qb + 8 * i);
      } else {
        reinterpret_cast<float4*>(rb + cur * row_elems + 8 * i)[0] = reinterpret_cast<const float4*>(qb + 8 * i)[0];
        reinterpret_cast<float4*>(rb + cur * row_elems + 8 * i)[1] = reinterpret_cast<const float4*>(qb + 8 * i)[1];
      }
    }
    __shared__ float sh[QS_PH][D_ROW];
    if (cond) {  // workgroup-uniform
      // summary query: thread (chunk ch, phase ph < QS_PH) sums rows ph,
      // ph + QS_PH, ... of the g*H rows (row r = ring row r / H, head r % H);
      // the phases are added in phase order
      if (ph < QS_PH) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const int rows = G * H;
        for (int r0 = ph; r0 < rows; r0 += 8 * QS_PH) {
          float v[8][8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int r = r0 + u * QS_PH;
            if (r < rows) {
              const int slot = r / H, h = r - slot * H;
              const TQ* src = slot == cur ? qb + h * D_ROW : rb + slot * row_elems + h * D_ROW;
              load8_f32(src + ch * 8, v[u]);
            } else {
#pragma unroll
              for (int k = 0; k < 8; ++k) v[u][k] = 0.f;
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] += v[u][k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) sh[ph][ch * 8 + k] = acc[k];
      }
      __syncthreads();
      if (t < 64) {  // wave 0 condenses group m
        const int lane = t;
        const float inv = 1.0f / (float)(G * H);
        float qc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float sum = sh[0][8 * lane + k];
          for (int p = 1; p < QS_PH; ++p) sum += sh[p][8 * lane + k];
          qc[k] = sum * inv;
        }
        float qr = sh[0][D_C + lane];
        for (int p = 1; p < QS_PH; ++p) qr += sh[p][D_C + lane];
        qr *= inv;
        const int64_t t0 = m * G;
        const int64_t page = table[(int64_t)b * table_stride + t0 / page_rows];
        const bf16_t* rows0 = pages + (page * page_rows + t0 % page_rows) * row_stride;
        RowChunk<bf16_t> rowsv[G];
        bf16_t krv[G];
#pragma unroll
        for (int r = 0; r < G; ++r) {
          rowsv[r].load(rows0 + r * row_stride + 8 * lane);
          krv[r] = __builtin_nontemporal_load(rows0 + r * row_stride + D_C + lane);
        }
        const GroupResult<bf16_t, LG> gr =
            condense_group<bf16_t, LG>(rowsv, krv, qc, qr, sm_scale, lane, LCA_MODE_LCA);
        bf16_t* dst = rc + (int64_t)b * rc_seq + m * rc_tok;
        store8(dst + 8 * lane, gr.acc);
        dst[D_C + lane] = (bf16_t)f2bf(gr.kval);
        if (lane == 0) anchor[(int64_t)b * anchor_seq + m] = (int32_t)(t0 + gr.arg);
      }
    }
    __syncthreads();  // every thread has read the state it is about to be replaced
    if (t == 0) {
      const int64_t mn = m + (cond ? 1 : 0), Ln = L + 1;
      seq_m[b] = (int32_t)mn;
      seq_raw_begin[b] = (int32_t)(mn * G);
      seq_raw_end[b] = (int32_t)Ln;
      if (pos != nullptr) pos[b] = (int32_t)Ln;
      if (dst_row != nullptr)
        dst_row[b] = Ln / page_rows < table_stride
                         ? (int64_t)table[(int64_t)b * table_stride + Ln / page_rows] * page_rows + Ln % page_rows
                         : -1;
    }
  }
};

template <class StepT>
__global__ __launch_bounds__(QS_THREADS) void condense_step_kernel(StepT st) {
  st.run((int)blockIdx.x);
}

// The step's arguments as the kernels take them.
template <typename TQ, int LG>
static CondenseStep<TQ, LG> make_step(const lca_paged_t& cache, int B, int64_t w, const void* q, int64_t q_seq_stride,
                                      int H, void* q_ring, int64_t q_ring_seq_stride, float sm_scale,
                                      const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq, int32_t* seq_m,
                                      int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos, int64_t* dst_row) {
  return CondenseStep<TQ, LG>{B, (const bf16_t*)cache.pages, cache.row_stride, cache.page_rows, cache.block_table,
                              cache.table_stride, w, (const TQ*)q, q_seq_stride, H, (TQ*)q_ring, q_ring_seq_stride,
                              sm_scale, (bf16_t*)reps.c, reps.c_seq_stride, reps.c_tok_stride, anchor, anchor_seq,
                              seq_m, seq_raw_begin, seq_raw_end, pos, dst_row};
}

// Dispatch on the query dtype and log2(g): F(step) is called with the
// step arguments of the matching instantiation.
template <class F>
static void with_step(int q_dtype, int g, const lca_paged_t& cache, int B, int64_t w, const void* q,
                      int64_t q_seq_stride, int H, void* q_ring, int64_t q_ring_seq_stride, float sm_scale,
                      const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq, int32_t* seq_m,
                      int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos, int64_t* dst_row, F&& f) {
  int lg = 0;
  while ((1 << lg) < g) ++lg;
#define LCA_STEP(TQV, LGV)                                                                                       \
  f(make_step<TQV, LGV>(cache, B, w, q, q_seq_stride, H, q_ring, q_ring_seq_stride, sm_scale, reps, anchor,      \
                        anchor_seq, seq_m, seq_raw_begin, seq_raw_end, pos, dst_row))
#define LCA_STEP_G(TQV)              \
  switch (lg) {                      \
    case 0: LCA_STEP(TQV, 0); break; \
    case 1: LCA_STEP(TQV, 1); break; \
    case 2: LCA_STEP(TQV, 2); break; \
    case 3: LCA_STEP(TQV, 3); break; \
    case 4: LCA_STEP(TQV, 4); break; \
    default: LCA_STEP(TQV, 5); break; \
  }
  if (q_dtype == LCA_BF16) {
    LCA_STEP_G(bf16_t)
  } else {
    LCA_STEP_G(float)
  }
#undef LCA_STEP_G
#undef LCA_STEP
}

hipError_t launch_condense_step(const lca_paged_t& cache, int B, int64_t w, int g, const void* q, int q_dtype,
                                int64_t q_seq_stride, int H, void* q_ring, int64_t q_ring_seq_stride,
                                float sm_scale, const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq,
                                int32_t* seq_m, int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos,
                                int64_t* dst_row, hipStream_t stream) {
  with_step(q_dtype, g, cache, B, w, q, q_seq_stride, H, q_ring, q_ring_seq_stride, sm_scale, reps, anchor,
            anchor_seq, seq_m, seq_raw_begin, seq_raw_end, pos, dst_row, [&](auto st) {
              hipLaunchKernelGGL((condense_step_kernel<decltype(st)>), dim3((unsigned)B), dim3(QS_THREADS), 0,
                                 stream, st);
            });
  return hipGetLastError();
}

// The W_UV up-projection of a decode's rows (up_rows_kernel over the split
// partials, which it merges, or over the merged fp32 rows) with the step
// condensation appended as B more workgroups of the same launch: they run
// after the decode attention kernel, the last reader of the state they
// rewrite.
template <class Src>
static hipError_t up_rows_step(const Src& rows, int B, int H, const void* w_uv, int w_dtype, void* out,
                               int out_dtype, const lca_paged_t& cache, int64_t w, int g, const void* q,
                               int q_dtype, int64_t q_seq_stride, void* q_ring, int64_t q_ring_seq_stride,
                               float sm_scale, const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq,
                               int32_t* seq_m, int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos,
                               int64_t* dst_row, hipStream_t stream) {
  const unsigned n_up = (unsigned)(((B + UpShapeStep::R - 1) / UpShapeStep::R) * H * UpShapeStep::F);
  const dim3 grid(n_up + (unsigned)B);
  with_step(q_dtype, g, cache, B, w, q, q_seq_stride, H, q_ring, q_ring_seq_stride, sm_scale, reps, anchor,
            anchor_seq, seq_m, seq_raw_begin, seq_raw_end, pos, dst_row, [&](auto st) {
              using ST = decltype(st);
              if (w_dtype == LCA_BF16) {
                if (out_dtype == LCA_BF16)
                  hipLaunchKernelGGL((up_rows_kernel<Src, bf16_t, bf16_t, ST>), grid, dim3(64 * UPR_WAVES), 0,
                                     stream, rows, (int64_t)B, H, (const bf16_t*)w_uv, (bf16_t*)out, st);
                else
                  hipLaunchKernelGGL((up_rows_kernel<Src, bf16_t, float, ST>), grid, dim3(64 * UPR_WAVES), 0,
                                     stream, rows, (int64_t)B, H, (const bf16_t*)w_uv, (float*)out, st);
              } else {
                if (out_dtype == LCA_BF16)
                  hipLaunchKernelGGL((up_rows_kernel<Src, float, bf16_t, ST>), grid, dim3(64 * UPR_WAVES), 0,
                                     stream, rows, (int64_t)B, H, (const float*)w_uv, (bf16_t*)out, st);
                else
                  hipLaunchKernelGGL((up_rows_kernel<Src, float, float, ST>), grid, dim3(64 * UPR_WAVES), 0,
                                     stream, rows, (int64_t)B, H, (const float*)w_uv, (float*)out, st);
              }
            });
  return hipGetLastError();
}

hipError_t launch_up_rows_step(const float* part_o, const float* part_ml, int S, float* o_latent, float* lse,
                               int B, int H, const void* w_uv, int w_dtype, void* out, int out_dtype,
                               const lca_paged_t& cache, int64_t w, int g, const void* q, int q_dtype,
                               int64_t q_seq_stride, void* q_ring, int64_t q_ring_seq_stride, float sm_scale,
                               const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq, int32_t* seq_m,
                               int32_t* seq_raw_begin, int32_t* seq_raw_end, int32_t* pos, int64_t* dst_row,
                               hipStream_t stream) {
  if (S > 1)
    return up_rows_step(RowsFromSplits{part_o, part_ml, S, o_latent, lse}, B, H, w_uv, w_dtype, out, out_dtype,
                        cache, w, g, q, q_dtype, q_seq_stride, q_ring, q_ring_seq_stride, sm_scale, reps, anchor,
                        anchor_seq, seq_m, seq_raw_begin, seq_raw_end, pos, dst_row, stream);
  return up_rows_step(RowsFromLatent<float>{o_latent}, B, H, w_uv, w_dtype, out, out_dtype, cache, w, g, q, q_dtype,
                      q_seq_stride, q_ring, q_ring_seq_stride, sm_scale, reps, anchor, anchor_seq, seq_m,
                      seq_raw_begin, seq_raw_end, pos, dst_row, stream);
}

template <typename TC, typename TR, int LG>
static void launch_k1(dim3 grid, hipStream_t st, const lca_latent_t& cache, const float* qbar,
                      int per_group_q, int64_t n_q, int64_t gb, int64_t ng, float sm,
                      const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq,
                      float* alpha, int64_t alpha_seq, int mode) {
  hipLaunchKernelGGL((condense_kernel<TC, TR, LG>), grid, dim3(256), 0, st,
                     (const TC*)cache.c, (const TC*)cache.kr, cache.c_seq_stride,
                     cache.c_tok_stride, cache.kr_seq_stride, cache.kr_tok_stride, qbar,
                     per_group_q, n_q, gb, ng, sm, (TR*)reps.c, (TR*)reps.kr, reps.c_seq_stride,
                     reps.c_tok_stride, reps.kr_seq_stride, reps.kr_tok_stride, anchor,
                     anchor_seq, alpha, alpha_seq, mode);
}

template <typename TC, typename TR>
static void dispatch_g(int lg, dim3 grid, hipStream_t st, const lca_latent_t& cache,
                       const float* qbar, int pg, int64_t n_q, int64_t gb, int64_t ng, float sm,
                       const lca_latent_t& reps, int32_t* anchor, int64_t as, float* alpha,
                       int64_t als, int mode) {
  switch (lg) {
    case 0: launch_k1<TC, TR, 0>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als, mode); break;
    case 1: launch_k1<TC, TR, 1>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als, mode); break;
    case 2: launch_k1<TC, TR, 2>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als, mode); break;
    case 3: launch_k1<TC, TR, 3>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als, mode); break;
    case 4: launch_k1<TC, TR, 4>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als, mode); break;
    default: launch_k1<TC, TR, 5>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als, mode); break;
  }
}

static void launch_qbar_shared(int B, int g, const void* q, int q_dtype, int64_t q_seq_stride,
                               int64_t q_tok_stride, int H, int64_t q_row0, float* qbar_ws, hipStream_t stream,
                               bool final_pass = true) {
  // workspace: [B][576] summary queries, then [B][QBAR_PARTS][576] part sums
  float* part = qbar_ws + (int64_t)B * D_ROW;
  dim3 gp((unsigned)QBAR_PARTS, (unsigned)B);
  if (q_dtype == LCA_BF16)
    hipLaunchKernelGGL(qbar_part_kernel<bf16_t>, gp, dim3(QP_THREADS), 0, stream, (const bf16_t*)q,
                       q_seq_stride, q_tok_stride, H, g, q_row0, part);
  else
    hipLaunchKernelGGL(qbar_part_kernel<float>, gp, dim3(QP_THREADS), 0, stream, (const float*)q,
                       q_seq_stride, q_tok_stride, H, g, q_row0, part);
  if (final_pass)
    hipLaunchKernelGGL(qbar_final_kernel, dim3((unsigned)B), dim3(D_ROW), 0, stream, part, g * H, qbar_ws);
}

hipError_t launch_condense_paged(const lca_paged_t& cache, int B, int g, const int32_t* seq_group_begin,
                                 const int32_t* seq_n_groups, int64_t max_groups, const void* q, int q_dtype,
                                 int64_t q_seq_stride, int64_t q_tok_stride, int H, int64_t q_row0,
                                 int64_t q_row_step, float sm_scale, const lca_latent_t& reps, int32_t* anchor,
                                 int64_t anchor_seq, float* alpha, int64_t alpha_seq, float* qbar_ws,
                                 hipStream_t stream) {
  // summary queries: one per sequence (decode), or one per group slot n <
  // max_groups (rows q_row0 + n q_row_step, the queries after each group in
  // chunked prefill); slots past a sequence's group count are not used
  const int per_group_q = q_row_step != 0;
  const int64_t n_q = per_group_q ? max_groups : 1;
  if (per_group_q) {
    dim3 g0((unsigned)n_q, (unsigned)B);
    if (q_dtype == LCA_BF16)
      hipLaunchKernelGGL(qbar_kernel<bf16_t>, g0, dim3(QBAR_THREADS), 0, stream, (const bf16_t*)q,
                         q_seq_stride, q_tok_stride, H, g, q_row0, q_row_step, (int)n_q, qbar_ws);
    else
      hipLaunchKernelGGL(qbar_kernel<float>, g0, dim3(QBAR_THREADS), 0, stream, (const float*)q,
                         q_seq_stride, q_tok_stride, H, g, q_row0, q_row_step, (int)n_q, qbar_ws);
  } else {
    launch_qbar_shared(B, g, q, q_dtype, q_seq_stride, q_tok_stride, H, q_row0, qbar_ws, stream);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int lg = 0;
  while ((1 << lg) < g) ++lg;
  dim3 grid((unsigned)((max_groups + 3) / 4), (unsigned)B);
#define LCA_PAGED(LGV)                                                                                     \
  hipLaunchKernelGGL((condense_paged_kernel<LGV>), grid, dim3(256), 0, stream, (const bf16_t*)cache.pages,   \
                     cache.row_stride, cache.page_rows, cache.block_table, cache.table_stride, seq_group_begin, \
                     seq_n_groups, qbar_ws, per_group_q, n_q, sm_scale, (bf16_t*)reps.c, reps.c_seq_stride,     \
                     reps.c_tok_stride,                                                                      \
                     anchor, anchor_seq, alpha, alpha_seq)
  switch (lg) {
    case 0: LCA_PAGED(0); break;
    case 1: LCA_PAGED(1); break;
    case 2: LCA_PAGED(2); break;
    case 3: LCA_PAGED(3); break;
    case 4: LCA_PAGED(4); break;
    default: LCA_PAGED(5); break;
  }
#undef LCA_PAGED
  return hipGetLastError();
}

hipError_t launch_condense(const lca_latent_t& cache, int B, int g, int64_t group_begin,
                           int64_t n_groups, const void* q, int q_dtype, int64_t q_seq_stride,
                           int64_t q_tok_stride, int H, int64_t q_row0, int64_t q_row_step,
                           float sm_scale, const lca_latent_t& reps, int32_t* anchor,
                           int64_t anchor_seq, float* alpha, int64_t alpha_seq, float* qbar_ws,
                           int mode, hipStream_t stream) {
  const int per_group_q = q_row_step != 0;
  const int64_t n_q = per_group_q ? n_groups : 1;
  if (per_group_q) {
    dim3 g0((unsigned)n_q, (unsigned)B);
    if (q_dtype == LCA_BF16)
      hipLaunchKernelGGL(qbar_kernel<bf16_t>, g0, dim3(QBAR_THREADS), 0, stream, (const bf16_t*)q,
                         q_seq_stride, q_tok_stride, H, g, q_row0, q_row_step, (int)n_q, qbar_ws);
    else
      hipLaunchKernelGGL(qbar_kernel<float>, g0, dim3(QBAR_THREADS), 0, stream, (const float*)q,
                         q_seq_stride, q_tok_stride, H, g, q_row0, q_row_step, (int)n_q, qbar_ws);
  }
  int lg = 0;
  while ((1 << lg) < g) ++lg;
  const bool packed = cache.dtype == LCA_BF16 && reps.dtype == LCA_BF16 &&
                      static_cast<const char*>(cache.kr) == static_cast<const char*>(cache.c) + 2 * D_C &&
                      cache.kr_tok_stride == cache.c_tok_stride && cache.kr_seq_stride == cache.c_seq_stride &&
                      cache.c_tok_stride * 2 * 32 < ((int64_t)1 << 31);
  const bool ring = mode == LCA_MODE_LCA && !per_group_q && packed && (lg == 3 || lg == 4) && n_groups > 0;
  if (!per_group_q)  // part sums, then the final pass unless the streaming kernel adds them itself
    launch_qbar_shared(B, g, q, q_dtype, q_seq_stride, q_tok_stride, H, q_row0, qbar_ws, stream, !ring);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (ring) {
    // one resident workgroup per CU; the waves of a sequence share its groups.
    // Sequences along x: a sequence's workgroups are B apart in dispatch
    // order, so for B a multiple of the 8 XCDs they all run on one XCD
    // (measured 0.7% faster than spreading each sequence over all XCDs at
    // B = 32 x 32K, outputs bitwise equal).
    const int64_t wpb = B >= 256 ? 1 : (256 + B - 1) / B;  // workgroups per sequence
    const int64_t nblk = std::min(wpb, (n_groups + 3) / 4);
    dim3 gr((unsigned)B, (unsigned)nblk);
#define LCA_RING(LGV, AL)                                                                          \
  hipLaunchKernelGGL((condense_ring_kernel<LGV, AL>), gr, dim3(256), 0, stream,                    \
                     static_cast<const char*>(cache.c), cache.c_seq_stride * 2, cache.c_tok_stride * 2, \
                     qbar_ws + (int64_t)B * D_ROW, g * H, group_begin, n_groups, sm_scale, (bf16_t*)reps.c, \
                     (bf16_t*)reps.kr, reps.c_seq_stride, reps.c_tok_stride, reps.kr_seq_stride,     \
                     reps.kr_tok_stride, anchor, anchor_seq, alpha, alpha_seq)
    if (lg == 3) { if (alpha) LCA_RING(3, true); else LCA_RING(3, false); }
    else { if (alpha) LCA_RING(4, true); else LCA_RING(4, false); }
#undef LCA_RING
    return hipGetLastError();
  }
  dim3 g1((unsigned)((n_groups + 3) / 4), (unsigned)B);
  const bool cb = cache.dtype == LCA_BF16, rb = reps.dtype == LCA_BF16;
  if (cb && rb)
    dispatch_g<bf16_t, bf16_t>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq, mode);
  else if (cb)
    dispatch_g<bf16_t, float>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq, mode);
  else if (rb)
    dispatch_g<float, bf16_t>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq, mode);
  else
    dispatch_g<float, float>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq, mode);
  return hipGetLastError();
}

}  // namespace lca
