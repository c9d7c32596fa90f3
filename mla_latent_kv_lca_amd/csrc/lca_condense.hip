// LCA condensation kernels for gfx950.
//
// Method: "Latent-Condensed Transformer for Efficient Long Context Modeling",
// 关键设计 1 (summary query = mean of the most recent g queries, per-token
// importance, softmax weights, weighted pooling of c_KV) and 关键设计 2 (the
// group's k_R is the k_R of its most important token).
//
// Two kernels:
//  qbar_kernel      one workgroup per summary query: mean over g query tokens
//                   and H heads of 576-wide absorbed queries -> fp32 workspace.
//  condense_kernel  one wavefront per group. Lane l owns latent columns
//                   [8l, 8l+8) and RoPE column l of all g rows, so each row
//                   load is one fully coalesced 1 KB (c_KV) + 128 B (k_R)
//                   wave access and every row's score is formed by the same
//                   sequence of operations (identical rows give bitwise equal
//                   scores). The g partial dot products are reduced across
//                   the 64 lanes with a halving butterfly (g/2 + g/4 + ...
//                   shuffles instead of 6 g), the g-way softmax / argmax uses
//                   shuffles, and the pooled row is accumulated in fp32.
// The work is HBM streaming (about 2 flop per byte): no matrix cores.
#include "lca_device.h"
#include "lca_internal.h"
#include "lca_stream.h"

namespace lca {

// ---------------------------------------------------------------- K0 -------
constexpr int QBAR_PH = 14;                  // row phases
constexpr int QBAR_THREADS = 72 * QBAR_PH;   // 72 column chunks of 8 x 14 row phases

// One workgroup per summary query: thread (chunk c, phase p) sums rows
// p, p + 14, ... of the g*H query rows, eight loads in flight at a time; the
// 14 phase partials are then added in phase order.
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

// ---------------------------------------------------------------- K1 -------
// v_cndmask with the lane mask in an SGPR pair, kept opaque: written as a C
// select, the compiler turns "upper ? v[i] : v[i + half]" into a variable
// index into v, which it then expands into a compare-and-select per element.
__device__ __forceinline__ float lane_select(uint64_t take_b, float a, float b) {
  float r;
  asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(take_b));
  return r;
}

// Reduce v[0..G) over all 64 lanes; afterwards every lane holds the total of
// row (lane >> (6 - LG)).
template <int LG>
__device__ __forceinline__ float reduce_rows(float (&v)[1 << LG], int lane) {
  constexpr int G = 1 << LG;
#pragma unroll
  for (int st = 0; st < LG; ++st) {
    const int mask = 32 >> st;
    const int half = G >> (st + 1);
    const uint64_t upper = __builtin_amdgcn_ballot_w64((lane & mask) != 0);
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = lane_select(upper, v[i + half], v[i]);  // upper lanes send v[i]
      const float keep = lane_select(upper, v[i], v[i + half]);
      v[i] = keep + __shfl_xor(send, mask);
    }
  }
  float x = v[0];
#pragma unroll
  for (int mask = 32 >> LG; mask >= 1; mask >>= 1) x += __shfl_xor(x, mask);
  return x;
}

template <typename TC> struct RowChunk;  // 8 latent elements of one row held by a lane
template <> struct RowChunk<bf16_t> {
  uint4 v;
  __device__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ float get(int i) const {
    const uint32_t w = u4_get(v, i >> 1);
    return (i & 1) ? bf_hi(w) : bf_lo(w);
  }
};
template <> struct RowChunk<float> {
  float v[8];
  __device__ void load(const float* p) { load8_f32(p, v); }
  __device__ float get(int i) const { return v[i]; }
};

// Scores, weights and pooled row of one group held by a wavefront (lane owns
// latent columns 8 lane .. 8 lane + 7 and RoPE column lane of every row).
// wsh: 32 floats of this wave's LDS, for the weights broadcast.
template <typename TC, int LG>
struct GroupResult {
  float acc[8];   // pooled latent columns of this lane
  int arg;        // anchor row within the group (wave-uniform)
  float a_mine;   // weight of row my_row
  int my_row;
  TC ksel;        // anchor row's RoPE column of this lane
};
template <typename TC, int LG>
__device__ __forceinline__ GroupResult<TC, LG> condense_group(const RowChunk<TC> (&rows)[1 << LG],
                                                             const TC (&krv)[1 << LG], const float (&qc)[8],
                                                             float qr, float sm_scale, int lane, float* wsh) {
  constexpr int G = 1 << LG;
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
  const float score = reduce_rows<LG>(s, lane);
  out.my_row = lane >> (6 - LG);
  // group max and first argmax over rows (rows sit in the top LG lane bits)
  float mx = score;
  int arg = out.my_row;
#pragma unroll
  for (int st = 0; st < LG; ++st) {
    const int mask = 32 >> st;
    const float om = __shfl_xor(mx, mask);
    const int oa = __shfl_xor(arg, mask);
    if (om > mx || (om == mx && oa < arg)) { mx = om; arg = oa; }
  }
  out.arg = __builtin_amdgcn_readfirstlane(arg);
  const float e = __expf(sm_scale * (score - mx));
  float tot = e;
#pragma unroll
  for (int st = 0; st < LG; ++st) tot += __shfl_xor(tot, 32 >> st);
  out.a_mine = e / tot;
  // every lane needs all G weights: one lane per row publishes its weight
  if ((lane & ((64 >> LG) - 1)) == 0) wsh[out.my_row] = out.a_mine;
  float al[G];
#pragma unroll
  for (int r = 0; r < G; ++r) al[r] = wsh[r];
  // pooled latent: sum_r alpha_r c_r in row order
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) out.acc[i] = (r == 0) ? al[r] * rows[r].get(i) : fmaf(al[r], rows[r].get(i), out.acc[i]);
  out.ksel = krv[0];
#pragma unroll
  for (int r = 1; r < G; ++r)
    if (r == out.arg) out.ksel = krv[r];  // arg is uniform: a scalar branch per row
  return out;
}

template <typename TC, typename TR, int LG>
__global__ __launch_bounds__(256) void condense_kernel(
    const TC* __restrict__ c, const TC* __restrict__ kr, int64_t c_seq, int64_t c_tok,
    int64_t kr_seq, int64_t kr_tok, const float* __restrict__ qbar, int per_group_q,
    int64_t n_q, int64_t group_begin, int64_t n_groups, float sm_scale, TR* __restrict__ rc,
    TR* __restrict__ rk, int64_t rc_seq, int64_t rc_tok, int64_t rk_seq, int64_t rk_tok,
    int32_t* __restrict__ anchor, int64_t anchor_seq, float* __restrict__ alpha,
    int64_t alpha_seq) {
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
    krv[r] = kg[r * kr_tok];
  }
  __shared__ float wsh[4][32];
  const GroupResult<TC, LG> gr = condense_group<TC, LG>(rows, krv, qc, qr, sm_scale, lane, wsh[threadIdx.x >> 6]);
  store8(rc + (int64_t)b * rc_seq + j * rc_tok + 8 * lane, gr.acc);
  rk[(int64_t)b * rk_seq + j * rk_tok + lane] = from_f32<TR>(to_f32(gr.ksel));
  if (lane == 0) anchor[(int64_t)b * anchor_seq + j] = (int32_t)(j * G + gr.arg);
  if (alpha != nullptr && (lane & ((64 >> LG) - 1)) == 0)
    alpha[(int64_t)b * alpha_seq + j * G + gr.my_row] = gr.a_mine;
}

// ---------------------------------------------------------------- K1r ------
// Streaming variant for packed bf16 rows and one summary query per sequence
// (decode-time condensation), g = 8 or 16. Each wavefront walks a contiguous
// run of groups of one sequence; group tiles (g rows x 1,152 bytes) stream
// from HBM straight into a wave-private LDS ring by direct loads, so the
// next groups are in flight while one is scored and pooled, and the
// workgroups stay resident instead of being re-dispatched per group.
// The arithmetic per group is exactly that of condense_kernel (same operand
// order), so both kernels give bitwise equal results.
// Completion of a tile is tracked with vmcnt, which also counts this wave's
// stores: every group issues exactly NST stores (pooled row, anchor k_R,
// anchor index, and the weights when requested), after the loads of the tile
// that reuses its slot.
template <int LG>
struct RingCfg {
  static constexpr int G = 1 << LG;
  static constexpr int TILE = G * D_ROW;                      // bf16 elements per group tile
  static constexpr int NS = LG == 3 ? 4 : 2;                  // slots per wave
  static constexpr int NI = G * (D_ROW / 8) / 64;             // load instructions per tile
};
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

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
    const char* __restrict__ cache, int64_t seq_b, int64_t tok_b, const float* __restrict__ qbar,
    int64_t group_begin, int64_t n_groups, int64_t per_wave, float sm_scale,
    bf16_t* __restrict__ rc, bf16_t* __restrict__ rk, int64_t rc_seq, int64_t rc_tok,
    int64_t rk_seq, int64_t rk_tok, int32_t* __restrict__ anchor, int64_t anchor_seq,
    float* __restrict__ alpha, int64_t alpha_seq) {
  using Cfg = RingCfg<LG>;
  constexpr int G = Cfg::G, NS = Cfg::NS, NI = Cfg::NI;
  __shared__ __align__(16) bf16_t ring[4][NS][Cfg::TILE];
  __shared__ float wsh[4][32];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int64_t first = ((int64_t)blockIdx.x * 4 + w) * per_wave;
  const int64_t last = min(n_groups, first + per_wave);
  if (first >= last) return;  // wave-uniform; the kernel has no barriers

  const float* qb = qbar + (int64_t)b * D_ROW;
  float qc[8];
  load8_f32(qb + 8 * lane, qc);
  const float qr = qb[D_C + lane];
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
  auto issue = [&](int64_t n) {
    const char* g0 = seq + (group_begin + n) * G * tok_b;
    const uint32_t base = lds_off(&ring[w][n % NS][0]);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(g0 + off[i], base + 1024u * i);
  };
#pragma unroll
  for (int k = 0; k < NS; ++k)
    if (first + k < last) issue(first + k);

  for (int64_t n = first; n < last; ++n) {
    // after tile n was issued: the stores of groups max(first, n - NS) .. n - 1
    // and the tiles n + 1 .. n + NS - 1
    wait_tile<LG, ALPHA>((int)min(n - first, (int64_t)NS), (int)min(last - 1 - n, (int64_t)NS - 1));
    const bf16_t* tile = &ring[w][n % NS][0];
    RowChunk<bf16_t> rows[G];
    bf16_t krv[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      rows[r].v = *reinterpret_cast<const uint4*>(tile + r * D_ROW + 8 * lane);
      krv[r] = tile[r * D_ROW + D_C + lane];
    }
    // the rows are in registers: the slot takes group n + NS right away
    if (n + NS < last) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(n + NS);
    }
    const int64_t j = group_begin + n;
    const GroupResult<bf16_t, LG> gr = condense_group<bf16_t, LG>(rows, krv, qc, qr, sm_scale, lane, wsh[w]);
    // exactly NST vector stores per group (counted by wait_tile)
    store8(rc + (int64_t)b * rc_seq + j * rc_tok + 8 * lane, gr.acc);
    rk[(int64_t)b * rk_seq + j * rk_tok + lane] = gr.ksel;
    if (lane == 0) anchor[(int64_t)b * anchor_seq + j] = (int32_t)(j * G + gr.arg);
    if (ALPHA && (lane & ((64 >> LG) - 1)) == 0) alpha[(int64_t)b * alpha_seq + j * G + gr.my_row] = gr.a_mine;
  }
}

template <typename TC, typename TR, int LG>
static void launch_k1(dim3 grid, hipStream_t st, const lca_latent_t& cache, const float* qbar,
                      int per_group_q, int64_t n_q, int64_t gb, int64_t ng, float sm,
                      const lca_latent_t& reps, int32_t* anchor, int64_t anchor_seq,
                      float* alpha, int64_t alpha_seq) {
  hipLaunchKernelGGL((condense_kernel<TC, TR, LG>), grid, dim3(256), 0, st,
                     (const TC*)cache.c, (const TC*)cache.kr, cache.c_seq_stride,
                     cache.c_tok_stride, cache.kr_seq_stride, cache.kr_tok_stride, qbar,
                     per_group_q, n_q, gb, ng, sm, (TR*)reps.c, (TR*)reps.kr, reps.c_seq_stride,
                     reps.c_tok_stride, reps.kr_seq_stride, reps.kr_tok_stride, anchor,
                     anchor_seq, alpha, alpha_seq);
}

template <typename TC, typename TR>
static void dispatch_g(int lg, dim3 grid, hipStream_t st, const lca_latent_t& cache,
                       const float* qbar, int pg, int64_t n_q, int64_t gb, int64_t ng, float sm,
                       const lca_latent_t& reps, int32_t* anchor, int64_t as, float* alpha,
                       int64_t als) {
  switch (lg) {
    case 0: launch_k1<TC, TR, 0>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    case 1: launch_k1<TC, TR, 1>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    case 2: launch_k1<TC, TR, 2>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    case 3: launch_k1<TC, TR, 3>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    case 4: launch_k1<TC, TR, 4>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
    default: launch_k1<TC, TR, 5>(grid, st, cache, qbar, pg, n_q, gb, ng, sm, reps, anchor, as, alpha, als); break;
  }
}

hipError_t launch_condense(const lca_latent_t& cache, int B, int g, int64_t group_begin,
                           int64_t n_groups, const void* q, int q_dtype, int64_t q_seq_stride,
                           int64_t q_tok_stride, int H, int64_t q_row0, int64_t q_row_step,
                           float sm_scale, const lca_latent_t& reps, int32_t* anchor,
                           int64_t anchor_seq, float* alpha, int64_t alpha_seq, float* qbar_ws,
                           hipStream_t stream) {
  const int per_group_q = q_row_step != 0;
  const int64_t n_q = per_group_q ? n_groups : 1;
  dim3 g0((unsigned)n_q, (unsigned)B);
  if (q_dtype == LCA_BF16)
    hipLaunchKernelGGL(qbar_kernel<bf16_t>, g0, dim3(QBAR_THREADS), 0, stream, (const bf16_t*)q,
                       q_seq_stride, q_tok_stride, H, g, q_row0, q_row_step, (int)n_q, qbar_ws);
  else
    hipLaunchKernelGGL(qbar_kernel<float>, g0, dim3(QBAR_THREADS), 0, stream, (const float*)q,
                       q_seq_stride, q_tok_stride, H, g, q_row0, q_row_step, (int)n_q, qbar_ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  int lg = 0;
  while ((1 << lg) < g) ++lg;
  const bool packed = cache.dtype == LCA_BF16 && reps.dtype == LCA_BF16 &&
                      static_cast<const char*>(cache.kr) == static_cast<const char*>(cache.c) + 2 * D_C &&
                      cache.kr_tok_stride == cache.c_tok_stride && cache.kr_seq_stride == cache.c_seq_stride &&
                      cache.c_tok_stride * 2 * 32 < ((int64_t)1 << 31);
  if (!per_group_q && packed && (lg == 3 || lg == 4) && n_groups > 0) {
    // one resident workgroup per CU: 4 waves x contiguous runs of groups
    const int64_t wpb = B >= 256 ? 1 : (256 + B - 1) / B;  // workgroups per sequence
    const int64_t per_wave = (n_groups + 4 * wpb - 1) / (4 * wpb);
    const int64_t nblk = (n_groups + 4 * per_wave - 1) / (4 * per_wave);
    dim3 gr((unsigned)nblk, (unsigned)B);
#define LCA_RING(LGV, AL)                                                                          \
  hipLaunchKernelGGL((condense_ring_kernel<LGV, AL>), gr, dim3(256), 0, stream,                    \
                     static_cast<const char*>(cache.c), cache.c_seq_stride * 2, cache.c_tok_stride * 2, \
                     qbar_ws, group_begin, n_groups, per_wave, sm_scale, (bf16_t*)reps.c,           \
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
    dispatch_g<bf16_t, bf16_t>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq);
  else if (cb)
    dispatch_g<bf16_t, float>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq);
  else if (rb)
    dispatch_g<float, bf16_t>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq);
  else
    dispatch_g<float, float>(lg, g1, stream, cache, qbar_ws, per_group_q, n_q, group_begin, n_groups, sm_scale, reps, anchor, anchor_seq, alpha, alpha_seq);
  return hipGetLastError();
}

}  // namespace lca
