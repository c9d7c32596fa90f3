// Streaming of packed latent rows from HBM straight into LDS, shared by the
// decode and prefill kernels (gfx950).
//
// A tile is 32 consecutive attended entries (representative rows first, then
// raw cache rows), stored densely in LDS (576 bf16 per row) with the 16-byte
// chunk c of row r at chunk position c ^ swz(r) (swz below): the rows read by
// one MFMA fragment then fall on distinct LDS banks. A workgroup of 4
// wavefronts fills a tile with 36 global_load_lds_dwordx4 wave instructions
// (16 bytes per lane straight into LDS, no register staging), 9 per wave.
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
// position c ^ swz(r). LDS has 64 banks of 4 bytes, and a row is 288 bank
// words, so rows of one parity start on bank 0 and the others on bank 32; a
// 16-byte read serves 16 lanes per pass and an 8-byte read 32. swz(r) is bits
// 1..3 of r in reverse order, which makes every access pattern of the kernels
// use each bank once per pass:
//  - K fragments (16 consecutive rows, one chunk each): the 8 rows of each
//    parity get 8 distinct values;
//  - decode's transposed V reads (8 aligned rows x 2 adjacent chunks): the 4
//    rows of each parity differ in bits 1-2;
//  - prefill's transposed V reads (4 aligned rows x 4 adjacent chunks): the 2
//    rows of each parity differ in bit 2.
// swz(r) depends on r mod 16 only.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1); }
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
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) dma16(b0 + off[i], base + 1024u * (w + SNW * i));
  } else {
    const int valid = (int)min((int64_t)STILE, e_end - e0);
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      int row, col;
      slot_rowcol(w, i, lane, row, col);
      const int64_t e = e0 + min(row, valid - 1);
      const char* p = e < src.m ? src.rep + e * src.tok : src.raw + (e - src.m) * src.tok;
      dma16(p + 16 * col, base + 1024u * (w + SNW * i));
    }
  }
}

}  // namespace lca
