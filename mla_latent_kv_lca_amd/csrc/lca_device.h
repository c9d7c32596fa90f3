// Device helpers shared by the gfx950 kernels: bf16 packing, vector loads and
// MFMA operand types. Nothing here is exported from the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lca {

constexpr int D_C = 512;           // latent c_KV width
constexpr int D_R = 64;            // decoupled RoPE key width
constexpr int D_ROW = D_C + D_R;   // one cached row
constexpr int D_V = 128;           // per-head value width after W_UV
constexpr int HB = 16;             // heads per MFMA block (the M/N extent of a 16x16 tile)

typedef uint16_t bf16_t;           // raw bfloat16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two floats -> two packed bfloat16 (lo in the low half), round to nearest
// even, NaN stays NaN: one v_cvt_pk_bf16_f32. (Written as integer rounding
// with a NaN test instead, the compiler emits a branch per element.)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f2bf(float f) { return pack_bf2(f, 0.f) & 0xffffu; }

// 8 consecutive elements of a bf16 or f32 array as 8 packed bf16 (one 16-byte
// operand fragment). p is 16-byte aligned for bf16, 32-byte for f32.
__device__ __forceinline__ uint4 load8_bf16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 load8_bf16(const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  return make_uint4(pack_bf2(a.x, a.y), pack_bf2(a.z, a.w), pack_bf2(b.x, b.y), pack_bf2(b.z, b.w));
}
// 4 consecutive elements as 4 packed bf16 (8 bytes).
__device__ __forceinline__ uint2 load4_bf16(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint2 load4_bf16(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  return make_uint2(pack_bf2(a.x, a.y), pack_bf2(a.z, a.w));
}

// 8 consecutive elements widened to f32.
__device__ __forceinline__ void load8_f32(const bf16_t* p, float* o) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  o[0] = bf_lo(v.x); o[1] = bf_hi(v.x); o[2] = bf_lo(v.y); o[3] = bf_hi(v.y);
  o[4] = bf_lo(v.z); o[5] = bf_hi(v.z); o[6] = bf_lo(v.w); o[7] = bf_hi(v.w);
}
__device__ __forceinline__ void load8_f32(const float* p, float* o) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// 8 consecutive elements kept in their stored type until converted, so that
// a batch of loads can be issued before any of them is used.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> { uint4 v; };
template <> struct Raw8<float> { float4 a, b; };
__device__ __forceinline__ Raw8<bf16_t> raw8_load(const bf16_t* p) {
  return Raw8<bf16_t>{*reinterpret_cast<const uint4*>(p)};
}
__device__ __forceinline__ Raw8<float> raw8_load(const float* p) {
  return Raw8<float>{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
}
template <typename T> __device__ __forceinline__ Raw8<T> raw8_zero();
template <> __device__ __forceinline__ Raw8<bf16_t> raw8_zero<bf16_t>() { return Raw8<bf16_t>{make_uint4(0u, 0u, 0u, 0u)}; }
template <> __device__ __forceinline__ Raw8<float> raw8_zero<float>() {
  return Raw8<float>{make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
}
__device__ __forceinline__ uint4 raw8_bf16(const Raw8<bf16_t>& r) { return r.v; }
__device__ __forceinline__ uint4 raw8_bf16(const Raw8<float>& r) {
  return make_uint4(pack_bf2(r.a.x, r.a.y), pack_bf2(r.a.z, r.a.w), pack_bf2(r.b.x, r.b.y), pack_bf2(r.b.z, r.b.w));
}

__device__ __forceinline__ float to_f32(bf16_t x) { return bf2f(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)f2bf(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Store 8 floats as 8 elements of T (16 or 32 bytes, aligned).
__device__ __forceinline__ void store8(bf16_t* p, const float* v) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                            pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
}
// Store 4 floats as 4 elements of T (8 or 16 bytes, aligned).
__device__ __forceinline__ void store4(bf16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// ---- MFMA wrappers (gfx950). Operand layouts for a 16x16 output tile:
//   16x16x32: lane l holds A[row l%16][k 8(l/16)..+7] and B[k 8(l/16)..+7][col l%16]
//   16x16x16: lane l holds A[row l%16][k 4(l/16)..+3] and B[k 4(l/16)..+3][col l%16]
//   result:   lane l holds D[row 4(l/16)+r][col l%16], r = 0..3
// Only the pairing of A's and B's k slots matters, so any consistent
// assignment of physical k to (lane group, element) gives the same product.
__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 32x32x16: lane l holds A[row l%32][k 8(l/32)..+7] and B[k 8(l/32)..+7][col l%32];
// the result D[row 8(r/4) + 4(l/32) + r%4][col l%32], r = 0..15.
__device__ __forceinline__ f32x16_t mfma32x32x16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16). The 16 lanes of each
// row group g (lanes 16 g .. 16 g + 15) each point at 4 consecutive 16-bit
// elements (8 bytes); lane 16 g + i receives element i % 4 of the rows
// pointed at by lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 of its group.
__device__ __forceinline__ uint2 lds_read_tr4(const bf16_t* p) {
  typedef short s16x4_lds __attribute__((ext_vector_type(4)));
  const s16x4_lds v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_lds*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Low / high bf16 halves of two words combined into one word: (lo(x), lo(y))
// or (hi(x), hi(y)). Used to turn row-major fragments into k-major operands.
__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) { return (x & 0xffffu) | (y << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) { return (x >> 16) | (y & 0xffff0000u); }

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

}  // namespace lca
