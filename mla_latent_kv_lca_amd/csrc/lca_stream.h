// Streaming of packed latent rows from HBM straight into LDS, shared by the
// decode and prefill kernels (gfx950).
//
// A tile is 32 consecutive attended entries (representative rows first, then
// raw cache rows), stored densely in LDS (576 bf16 per row) with the 16-byte
// chunk c of row r at chunk position c ^ swz(r) (swz below): the rows read by
// one MFMA fragment then fall on distinct LDS banks. Four wavefronts of the
// prefill workgroup fill a tile with 36 global_load_lds_dwordx4 wave
// instructions (16 bytes per lane straight into LDS, no register staging), 9
// per wave; the decode kernel's waves each load their own 16-row tiles.
#pragma once
#include "lca_tile.h"

namespace lca {

constexpr int STILE = 32;                                 // entries per tile
constexpr int SNW = 4;                                    // wavefronts filling a tile
constexpr int STILE_ELEMS = STILE * D_ROW;                // 36,864 bytes
constexpr int DMA_PER_WAVE = STILE * (D_ROW / 8) / 64 / SNW;  // 9 wave instructions

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
// Issued from asm so that the compiler does not drain the ring before every
// LDS read; completion is tracked with explicit vmcnt waits. m0 is saved and
// restored around the load, so the compiler's own use of m0 is untouched.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_block) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_block)
      : "memory");
}
// The same load marked non-temporal (streaming): for rows read exactly once,
// so they do not displace data that is read again.
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_block) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_block)
      : "memory");
}
// N direct loads of 16 bytes per lane: load i reads base + off[i] (base
// wave-uniform, off[i] a per-lane byte offset below 4 GiB that the load adds
// itself, so there is no 64-bit address arithmetic per load) into the LDS
// block lds0 + STEP i. Three loads per asm block with m0 saved once; the
// blocks step m0 with s_add_u32, which writes SCC (declared clobbered).
// readfirstlane returns int, so the uniform values pass through uint32_t and
// nothing is sign-extended into the 64-bit base.
#define LCA_DMA3(MOD)                                  \
  "s_mov_b32 %0, m0\n\t"                               \
  "s_mov_b32 m0, %4\n\t"                               \
  "global_load_lds_dwordx4 %1, %5" MOD "\n\t"          \
  "s_add_u32 m0, m0, %6\n\t"                           \
  "global_load_lds_dwordx4 %2, %5" MOD "\n\t"          \
  "s_add_u32 m0, m0, %6\n\t"                           \
  "global_load_lds_dwordx4 %3, %5" MOD "\n\t"          \
  "s_mov_b32 m0, %0"
template <uint32_t STEP, bool NT, int N>
__device__ __forceinline__ void dma16_rows(const void* base, const uint32_t (&off)[N], uint32_t lds0) {
  static_assert(N % 3 == 0, "three loads per asm block");
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t b_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t b_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t bu = ((uint64_t)b_hi << 32) | (uint64_t)b_lo;
  const uint32_t l0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds0);
#pragma unroll
  for (int j = 0; j < N; j += 3) {
    uint32_t saved;
    if constexpr (NT)
      asm volatile(LCA_DMA3(" nt")
                   : "=&s"(saved)
                   : "v"(off[j]), "v"(off[j + 1]), "v"(off[j + 2]), "s"(l0 + STEP * (uint32_t)j), "s"(bu), "i"(STEP)
                   : "memory", "scc");
    else
      asm volatile(LCA_DMA3("")
                   : "=&s"(saved)
                   : "v"(off[j]), "v"(off[j + 1]), "v"(off[j + 2]), "s"(l0 + STEP * (uint32_t)j), "s"(bu), "i"(STEP)
                   : "memory", "scc");
  }
}
#undef LCA_DMA3

// wait until at most `newer` tiles issued after the one wanted are in flight
__device__ __forceinline__ void wait_dma_newer(int newer) {
  static_assert(DMA_PER_WAVE == 9, "vmcnt immediates assume 9 loads per tile per wave");
  if (newer >= 3) asm volatile("s_waitcnt vmcnt(27)" ::: "memory");
  else if (newer == 2) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else if (newer == 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// An empty asm that reads the four registers: the compiler must have waited
// for the load that produced them before this point.
__device__ __forceinline__ void retire(const uint4& v) {
  asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}

// Tile rows are dense (576 bf16); the 16-byte chunk c of row r sits at chunk
// position c ^ swz(r), swz(r) = r mod 8. The kernels read a tile in two
// patterns, both the operands of 16x16 MFMA tiles:
//  - K fragments: lane (g, i) of the four 16-lane groups reads chunk 4 s + g
//    of row i (16 rows, four adjacent chunks per row);
//  - transposed V reads (ds_read_b64_tr_b16): lane (g, i) points at row
//    4 g + i / 4, 8 bytes of two adjacent chunks (8 rows x 2 chunks per 32
//    lanes).
// With this swizzle both run without LDS bank conflicts (SQ_LDS_BANK_CONFLICT
// = 0 in a probe that reads a tile in each pattern). A swizzle built from
// bits 1..3 of r in reverse order, which suits 32x32 fragments, gives the
// K fragments two-way conflicts on gfx950 (about half of the LDS cycles).
// swz(r) depends on r mod 8, so rows r and r + 16 share it.
__device__ __forceinline__ int swz(int r) { return r & 7; }
__device__ __forceinline__ int chunk_pos(int r, int c) { return r * (D_ROW / 8) + (c ^ swz(r)); }

// Packed rows (k_R right after c_KV, one token stride) of the two segments of
// one sequence: entries [0, m) are representative rows, the rest raw rows.
struct DmaSrc {
  const char* rep;  // representative rows of sequence 0
  const char* raw;  // raw rows of sequence 0, starting at raw_begin
  int64_t tok;      // token stride in bytes, shared by both segments
  int64_t m;
};

// LDS slot P = 64 j + lane (j = w + SNW i) of a tile holds 16-byte chunk
// col = (P % 72) ^ swz(row) of tile row row = P / 72; its byte offset from
// the tile's first row is row * token stride + 16 col, fixed for every tile.
__device__ __forceinline__ void slot_rowcol(int w, int i, int lane, int& row, int& col) {
  const int P = 64 * (w + SNW * i) + lane;
  row = P / 72;
  col = (P - row * 72) ^ swz(row);
}

// Issue the DMA of tile entries [e0, e0 + STILE) into `buf`. Full tiles inside
// one segment use uniform row bases plus per-lane offsets; the tile that
// straddles the representative / raw boundary and the last, partial tile
// compute each row, reloading the last valid row past e_end (those logits
// are masked, so any finite row will do).
__device__ __forceinline__ void tile_dma(const DmaSrc& src, int64_t e0, int64_t e_end,
                                         const bf16_t* buf, int w, int lane,
                                         const uint32_t (&off)[DMA_PER_WAVE]) {
  const uint32_t base = lds_off(buf);
  if (e0 + STILE <= e_end && (e0 + STILE <= src.m || e0 >= src.m)) {
    const char* b0 = e0 < src.m ? src.rep + e0 * src.tok : src.raw + (e0 - src.m) * src.tok;
    dma16_rows<1024u * SNW, false>(b0, off, base + 1024u * w);
  } else {
    const int valid = (int)min((int64_t)STILE, e_end - e0);
#pragma unroll 1  // rare boundary tiles: keep the per-lane row arithmetic small
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      int row, col;
      slot_rowcol(w, i, lane, row, col);
      const int64_t e = e0 + min(row, valid - 1);
      const char* p = e < src.m ? src.rep + e * src.tok : src.raw + (e - src.m) * src.tok;
      dma16(p + 16 * col, base + 1024u * (w + SNW * i));
    }
  }
}

// The same tiles over a paged cache (one sequence): entries [0, m) are
// dense representative rows, entry e >= m is raw token t = raw_begin + e - m,
// row t % P of page table[t / P] of the pool (P rows per page, a multiple of
// 16, so a 32-entry tile touches at most three pages). Representatives and
// pages share one row stride.
struct PagedDmaSrc {
  const char* rep;      // representative rows
  const char* pages;    // page pool
  const int32_t* table; // this sequence's block table
  int64_t tok;          // row stride in bytes
  int64_t m, raw_begin;
  int P;                // rows per page
};

__device__ __forceinline__ void tile_dma(const PagedDmaSrc& src, int64_t e0, int64_t e_end,
                                         const bf16_t* buf, int w, int lane,
                                         const uint32_t (&off)[DMA_PER_WAVE]) {
  const uint32_t base = lds_off(buf);
  const int valid = (int)min((int64_t)STILE, e_end - e0);
  if (e0 + STILE <= src.m && valid == STILE) {  // whole tile of representatives
    dma16_rows<1024u * SNW, false>(src.rep + e0 * src.tok, off, base + 1024u * w);
    return;
  }
  // raw tokens of the tile's raw entries and their pages (page indices are
  // wave-uniform scalar loads)
  const int64_t r_first = max(e0, src.m), r_last = e0 + valid - 1;
  const int64_t t_first = src.raw_begin + (r_first - src.m), t_last = src.raw_begin + (r_last - src.m);
  const int64_t pg0 = t_first / src.P, pg_last = r_last >= src.m ? t_last / src.P : pg0;
  const int64_t pa = src.table[__builtin_amdgcn_readfirstlane((int)pg0)];
  const int64_t pb = src.table[__builtin_amdgcn_readfirstlane((int)min(pg0 + 1, pg_last))];
  const int64_t pc = src.table[__builtin_amdgcn_readfirstlane((int)min(pg0 + 2, pg_last))];
  if (e0 >= src.m && valid == STILE) {  // whole tile of raw rows
    const uint64_t b0 = (uint64_t)(uintptr_t)(src.pages + (pa * src.P + (t_first - pg0 * src.P)) * src.tok);
    if (pg0 == pg_last) {  // in one page
      dma16_rows<1024u * SNW, false>((const void*)(uintptr_t)b0, off, base + 1024u * w);
      return;
    }
    // across two or three pages: rows [0, k1) continue page pa, rows [k1,
    // k1 + P) are page pb, the rest page pc; each segment's base is shifted
    // back by its first row, so that base + row x stride addresses the row
    // inside its page (a rolled loop: the kernel's registers are spoken for)
    const int k1 = (int)(src.P - (t_first - pg0 * src.P));
    const uint64_t tok = (uint64_t)src.tok, p0 = (uint64_t)(uintptr_t)src.pages;
    const uint64_t b1 = p0 + (uint64_t)pb * src.P * tok - (uint64_t)k1 * tok;
    const uint64_t b2 = p0 + (uint64_t)pc * src.P * tok - (uint64_t)(k1 + src.P) * tok;
#pragma unroll 1
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      int row, col;
      slot_rowcol(w, i, lane, row, col);
      const uint64_t b = row < k1 ? b0 : (row < k1 + src.P ? b1 : b2);
      dma16((const void*)(uintptr_t)(b + (uint64_t)row * tok + 16u * col), base + 1024u * (w + SNW * i));
    }
    return;
  }
#pragma unroll 1  // rare boundary tiles: keep the per-lane row arithmetic small
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    int row, col;
    slot_rowcol(w, i, lane, row, col);
    const int64_t e = e0 + min(row, valid - 1);
    const char* p;
    if (e < src.m) {
      p = src.rep + e * src.tok;
    } else {
      const int64_t t = src.raw_begin + (e - src.m), pg = t / src.P;
      const int64_t page = pg == pg0 ? pa : (pg == pg0 + 1 ? pb : pc);
      p = src.pages + (page * src.P + (t - pg * src.P)) * src.tok;
    }
    dma16(p + 16 * col, base + 1024u * (w + SNW * i));
  }
}

}  // namespace lca
