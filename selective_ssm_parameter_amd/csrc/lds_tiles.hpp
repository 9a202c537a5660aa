// LDS tile helpers for the scan: buffer-to-LDS copies of row-major tiles with an
// XOR chunk swizzle, and K-major matrix-core fragments read back from them with
// the gfx950 transposing LDS read.
#pragma once

#include "common.hpp"

namespace swimba {

// Swizzles (16-byte chunk index XOR, 2-byte element types; none for fp32).
// Tiles read with transposing loads (X, B): a 16-lane group reads two adjacent
// chunks of 4 consecutive rows; groups g and g + 1 read rows 8 apart.
template <typename T, int CPR>
__device__ __forceinline__ int swz_tr(int r) {
  if constexpr (sizeof(T) != 2) return 0;
  else if constexpr (CPR >= 16) return 2 * ((r & 3) | ((r >> 1) & 4));
  else if constexpr (CPR == 8) return 2 * ((r & 3) ^ ((r >> 3) & 1));
  else return 2 * (((r >> 1) & 1) ^ ((r >> 3) & 1));
}
// Tiles read by rows (C~, G, GEMM operands): a 16-byte read per lane, lane
// (g, c) taking chunk g of row c of 16 rows (consecutive rows, or the GEMM's
// weight rows 8 (c / 4) + c % 4 (+ 4)). The XOR patterns are the ones the LDS
// bank-conflict counter of gfx950 reads as zero for these accesses (64-byte
// rows: ((t >> 1) ^ (t >> 2)) & 3, where t & 3 and (t >> 1) ^ (t >> 3) conflict;
// 128-byte rows: t & 7, where t ^ (t >> 3) conflicts).
template <typename T, int CPR>
__device__ __forceinline__ int swz_row(int t) {
  if constexpr (sizeof(T) != 2) return 0;
  else if constexpr (CPR >= 16) return t & 15;
  else if constexpr (CPR == 8) return t & 7;
  else return ((t >> 1) ^ (t >> 2)) & 3;
}

// Buffer-to-LDS copy of a row-major tile: NROWS rows of CPR 16-byte chunks,
// global row r at byte offset base + r * pitch, chunk c at + 16 c. Chunk c of
// row r lands at LDS byte (r * CPR + (c ^ swz(r))) * 16 of dst. Rows >= rvalid
// and chunks >= cvalid are read as zeros. Each instruction of a wave moves 64
// consecutive LDS chunks; the 4 waves take turns.
template <int NROWS, int CPR, class Swz>
__device__ __forceinline__ void dma_tile(BufRes rs, uint32_t base, uint32_t pitch,
                                         unsigned char* dst, int rvalid, int cvalid, int wave,
                                         int lane, Swz swz) {
  static_assert((NROWS * CPR) % 64 == 0, "tile must be whole 64-chunk groups");
  constexpr int NI = NROWS * CPR / 64;
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += 4) {
    const int i = i0 + wave;
    if (NI % 4 == 0 || i < NI) {
      const int slot = 64 * i + lane;
      const int r = slot / CPR, pc = slot % CPR;
      const int lc = pc ^ swz(r);
      const uint32_t off = (r < rvalid && lc < cvalid) ? base + r * pitch + 16 * lc : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, off, 0, 0, 0);
    }
  }
}

// Copies of a tile whose rows and chunks are all valid: each lane's byte
// offset within the tile is fixed (planned once), and the tile's position
// enters as the copy's scalar offset, so a copy costs no vector arithmetic.
// off[m] is the lane's offset for this wave's m-th instruction (instruction
// 4m + wave of the tile, as in dma_tile).
template <int NROWS, int CPR, class Swz>
__device__ __forceinline__ void dma_plan(uint32_t pitch, int wave, int lane, Swz swz,
                                         uint32_t* off) {
  constexpr int NI = NROWS * CPR / 64;
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += 4) {
    const int slot = 64 * (i0 + wave) + lane;
    const int r = slot / CPR, pc = slot % CPR;
    off[i0 / 4] = r * pitch + 16 * (pc ^ swz(r));
  }
}
template <int NROWS, int CPR>
__device__ __forceinline__ void dma_tile_full(BufRes rs, uint32_t base, const uint32_t* off,
                                              unsigned char* dst, int wave) {
  constexpr int NI = NROWS * CPR / 64;
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += 4) {
    const int i = i0 + wave;
    if (NI % 4 == 0 || i < NI) {
      const uint32_t o = off[i0 / 4];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, o, base, 0, 0);
    }
  }
}

// Copies of a tile shared by NWV waves in which every wave issues the same
// number of instructions (dma_count), so that a wave can wait for a tile with
// a fixed vector-memory count: instruction m of wave w moves the tile's
// 64-chunk group m NWV + w; when the group count NI is not a multiple of NWV,
// the waves past the last group repeat one already moved (the same bytes to
// the same LDS place).
template <int NROWS, int CPR, int NWV>
constexpr int dma_count() {
  return (NROWS * CPR / 64 + NWV - 1) / NWV;
}
template <int NROWS, int CPR, int NWV>
__device__ __forceinline__ int dma_group(int m, int wave) {
  constexpr int NI = NROWS * CPR / 64;
  const int i = m * NWV + wave;
  return i < NI ? i : i % NI;
}
template <int NROWS, int CPR, int NWV, class Swz>
__device__ __forceinline__ void dma_plan_n(uint32_t pitch, int wave, int lane, Swz swz,
                                           uint32_t* off) {
  static_assert((NROWS * CPR) % 64 == 0, "tile must be whole 64-chunk groups");
#pragma unroll
  for (int m = 0; m < dma_count<NROWS, CPR, NWV>(); ++m) {
    const int slot = 64 * dma_group<NROWS, CPR, NWV>(m, wave) + lane;
    const int r = slot / CPR, pc = slot % CPR;
    off[m] = r * pitch + 16 * (pc ^ swz(r));
  }
}
// Every row and chunk valid: per-lane offsets from dma_plan_n, the tile's
// position as the scalar offset.
template <int NROWS, int CPR, int NWV>
__device__ __forceinline__ void dma_tile_full_n(BufRes rs, uint32_t base, const uint32_t* off,
                                                unsigned char* dst, int wave) {
#pragma unroll
  for (int m = 0; m < dma_count<NROWS, CPR, NWV>(); ++m) {
    const int i = dma_group<NROWS, CPR, NWV>(m, wave);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, off[m], base, 0, 0);
  }
}
// dma_tile_full_n with this wave's LDS position given as a byte offset wl =
// 1024 * dma_group(0, wave) that the caller recomputes at each use (through an
// empty volatile asm): the compiler then forms every copy's LDS address from
// it inside the loop instead of keeping one scalar register per copy and stage
// live across the whole walk.
template <int NROWS, int CPR, int NWV>
__device__ __forceinline__ void dma_tile_full_w(BufRes rs, uint32_t base, const uint32_t* off,
                                                unsigned char* dst, int wl) {
  constexpr int NI = NROWS * CPR / 64, NC = dma_count<NROWS, CPR, NWV>();
  static_assert(NI % NWV == 0 || NC == 1, "group m of a wave lies NWV groups after group m - 1");
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(dst + wl + 1024 * NWV * m), 16, off[m], base,
        0, 0);
  }
}

// Rows >= rvalid and chunks >= cvalid read as zeros; the same instruction
// count as dma_tile_full_n.
template <int NROWS, int CPR, int NWV, class Swz>
__device__ __forceinline__ void dma_tile_n(BufRes rs, uint32_t base, uint32_t pitch,
                                           unsigned char* dst, int rvalid, int cvalid, int wave,
                                           int lane, Swz swz) {
#pragma unroll
  for (int m = 0; m < dma_count<NROWS, CPR, NWV>(); ++m) {
    const int i = dma_group<NROWS, CPR, NWV>(m, wave);
    const int slot = 64 * i + lane;
    const int r = slot / CPR, pc = slot % CPR;
    const int lc = pc ^ swz(r);
    const uint32_t off = (r < rvalid && lc < cvalid) ? base + r * pitch + 16 * lc : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, off, 0, 0, 0);
  }
}

// dma_tile_full_n with a row limit: the copy of instruction m reads zeros
// unless row[m] < rvalid (row[m]: the tile row, in the caller's numbering, of
// this lane's chunk; off[m] its offset within the tile).
template <int NROWS, int CPR, int NWV>
__device__ __forceinline__ void dma_rows_n(BufRes rs, uint32_t base, const uint32_t* off,
                                           const int* row, int rvalid, unsigned char* dst,
                                           int wave) {
#pragma unroll
  for (int m = 0; m < dma_count<NROWS, CPR, NWV>(); ++m) {
    const int i = dma_group<NROWS, CPR, NWV>(m, wave);
    const uint32_t o = row[m] < rvalid ? off[m] + base : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, o, 0, 0, 0);
  }
}

// A K-major operand fragment from a row-major [k][col] LDS tile: lane (g, c)
// gets rows k0 + 8g .. k0 + 8g + 7 of column col0 + c. 2-byte types use two
// transposing reads (in a 16-lane group, lane i receives element i % 4 of the
// 4-element row pieces addressed by lanes i / 4 + 4 m, m = 0..3); fp32 reads
// the 8 elements one by one.
template <typename T, int CPR>
__device__ __forceinline__ typename Vec<T>::x8 load_kmajor(const unsigned char* tile, int k0,
                                                           int col0, int lane) {
  typedef typename Vec<T>::x8 F;
  const int g = lane >> 4, c = lane & 15;
  F v;
  if constexpr (sizeof(T) == 2) {
    typedef short s4 __attribute__((__vector_size__(8)));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = k0 + 8 * g + 4 * hh + (c >> 2);
      const int col = col0 + 4 * (c & 3);                 // element column of this lane's piece
      const int ch = col >> 3, half = (col >> 2) & 1;      // 16-byte chunk, 8-byte half
      const unsigned char* p = tile + (r * CPR + (ch ^ swz_tr<T, CPR>(r))) * 16 + 8 * half;
      const typename Vec<T>::x4 w4 = __builtin_bit_cast(
          typename Vec<T>::x4,
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(p)));
#pragma unroll
      for (int m = 0; m < 4; ++m) v[4 * hh + m] = w4[m];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = k0 + 8 * g + j, col = col0 + c;
      v[j] = *reinterpret_cast<const T*>(tile + r * CPR * 16 + col * (int)sizeof(T));
    }
  }
  return v;
}

// s_waitcnt with only the vector-memory count limited to n (0 <= n < 64): the
// copies issued before the last n of this wave have landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for staged loops: waits for this wave's LDS accesses only
// (lgkmcnt), not for copies still in flight to other stages (each wave waits
// for the stage it needs with wait_vm first); the empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace swimba
