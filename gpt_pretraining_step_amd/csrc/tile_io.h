// Tile movement between HBM and LDS shared by the MFMA kernels.
//
//  * DMA: global_load_lds_dwordx4 copies 16 bytes per lane straight into LDS;
//    one wave instruction fills 1 KB of consecutive LDS bytes (lane l at byte
//    16 l from the wave's base).
//  * Swizzle: a tile row of BK bf16 elements is stored without padding, its
//    16-byte chunk c at position c ^ swz(row).  The LDS has 64 banks of 4
//    bytes (256 bytes per pass); a 16-byte read serves 16 lanes per pass
//    and an 8-byte (transposing) read 32.  For 128-byte rows two rows share
//    a pass's 256 bytes, so swz(row) must take 8 distinct values on the
//    even and on the odd rows of any 16 consecutive rows (the 16 lanes of a
//    row-fragment read), and rows r and r + 2 of a 4-row transposing read
//    must differ in bit 2: swz(row) = ((row >> 1) & 1) << 2 | (row >> 2) & 3.
//    (row & 7, the 32-bank choice, leaves every such read 2-way
//    conflicted.)
//  * Transposed operand reads: ds_read_b64_tr_b16 (gfx950).  Within each
//    group of 16 lanes, source lane j supplies the 8 bytes at its address and
//    result lane i receives element i%4 of the vectors of source lanes i/4,
//    i/4+4, i/4+8, i/4+12.  If source lane j points at row r0 + j/4, columns
//    c0 + 4 (j%4) .. +3 of a row-major tile, result lane i holds column c0 + i
//    of rows r0 .. r0+3: a column read of the tile.
#pragma once

#include "common.h"

namespace g2 {

// Out-of-range DMA lanes copy from this block of zeros, so ragged M, N and K
// tails read as zeros.

__device__ __attribute__((aligned(16))) static const uint4 g2_zero16[4] = {};

// ---- copies issued through inline asm.  The compiler's wait insertion does
// not see them, so it neither drains them before LDS reads it cannot prove
// disjoint (it does so, conservatively, before every transposing read that
// follows a copy it knows of) nor waits for them anywhere else: the caller
// orders them with s_waitcnt vmcnt and a barrier before any wave reads what
// they fill.  Each statement sets M0, the LDS byte address of lane 0's 16
// bytes (lane l writes at M0 + 16 l).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ uint32_t uniform32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// source = uniform base + per-lane 32-bit byte offset
__device__ __forceinline__ void dma16_off(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t sb = (uint64_t)uniform32((uint32_t)b) | ((uint64_t)uniform32((uint32_t)(b >> 32)) << 32);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(uniform32(lds))
               : "m0");
}
// source = per-lane 64-bit address
__device__ __forceinline__ void dma16_ptr(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(uniform32(lds)) : "m0");
}
// 4 bytes per lane (lane l writes at M0 + 4 l)
__device__ __forceinline__ void dma4_ptr(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(uniform32(lds)) : "m0");
}
#pragma clang diagnostic pop

// A wait on every vector-memory load that the compiler can see (through the
// builtin, so that it knows them complete afterwards).  Kernels whose main
// loop copies with the asm forms above call it before the loop: otherwise the
// compiler's wait for a load issued before the loop lands at its first use
// inside the loop and drains the in-flight copies on every iteration.
__device__ __forceinline__ void drain_vector_loads() { __builtin_amdgcn_s_waitcnt(0x0070); }  // vmcnt(0) lgkmcnt(0)

template <int BK>
__device__ __forceinline__ int swz_chunk(int row, int c) {
  static_assert(BK == 64, "128-byte tile rows");
  return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// K-major tile [ROWS][BK] (source rows row0.., K columns k0..) -> LDS, by DMA.
template <int ROWS, int BK, int NWAVES, bool ASM = false>
__device__ __forceinline__ void dma_rows(bf16* lds, const bf16* __restrict__ src, int64_t ld, int row0, int nrows,
                                         int k0, int K) {
  constexpr int CPR = BK / 8;              // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;            // rows per wave instruction
  constexpr int INSTR = ROWS / RPI;        // instructions per tile
  static_assert(ROWS % RPI == 0, "whole instructions");
  // an even split gives each wave a contiguous run of instructions; an
  // uneven one deals them out in turn (some waves issue one fewer)
  constexpr bool EVEN = INSTR % NWAVES == 0;
  constexpr int IPW = (INSTR + NWAVES - 1) / NWAVES;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / CPR, pc = lane % CPR;
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int ins = EVEN ? wave * IPW + i : wave + i * NWAVES;
    if (!EVEN && ins >= INSTR) break;
    const int r = ins * RPI + rl;
    const int c = swz_chunk<BK>(r, pc);
    const int gr = row0 + r, gk = k0 + 8 * c;
    const bf16* g = (gr < nrows && gk < K) ? src + (int64_t)gr * ld + gk : reinterpret_cast<const bf16*>(g2_zero16);
    if constexpr (ASM) dma16_ptr(g, lds_addr(lds + ins * RPI * BK));
    else __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g), lds + ins * RPI * BK, 16, 0, 0);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Column read of a swizzled [rows][64] tile (128-byte rows): returns for
// this lane column c0 + (lane % 16) of rows r0..r0+3 (r0 % 4 == 0, c0 % 16 == 0).
__device__ __forceinline__ bf16x4 tr_read4(const bf16* tile, int r0, int c0) {
  const int j = threadIdx.x & 15;
  const int row = r0 + (j >> 2);
  const int col = c0 + 4 * (j & 3);
  const int byte = row * 128 + (swz_chunk<64>(row, col >> 3) << 4) + ((col & 7) << 1);
  auto base = (__attribute__((address_space(3))) char*)(tile);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + byte));
  return __builtin_bit_cast(bf16x4, v);
}

// ---- tiles stored with K as the row index: [BK rows][R columns], R bf16 per
// row (the output rows of a product whose operand is K-slow in memory).
// One transposing read (32 lanes per pass) covers 4 rows x 4 chunks.  With
// rows of 512 bytes (R = 256; R = 128 likewise) every row starts on bank 0,
// so chunk c of row k sits at c ^ ((k & 3) << 2): the 4 rows use 4 disjoint
// 4-chunk groups.  With R = 192 or 64 the row stride alone staggers the
// rows over the banks and c ^ ((k & 3) << 1) is conflict-free.  The XOR
// stays inside the row (R / 8 a multiple of 16, resp. 8).
template <int R>
__device__ __forceinline__ int kr_chunk(int k, int c) {
  static_assert(R % 64 == 0, "rows of whole 8-chunk groups");
  if constexpr (R % 128 == 0) return c ^ ((k & 3) << 2);
  else return c ^ ((k & 3) << 1);
}

// [BK][R] tile (source rows k0.. of a [K][ld] matrix, columns col0..col0+R)
// -> LDS by DMA; rows past K and columns past ncols read as zeros.  Wave
// instruction i fills LDS chunks 64 i .. 64 i + 63 of the tile (chunk g is
// row g / (R/8), position g % (R/8)); the lane whose destination is position
// p of row k fetches the logical chunk that the swizzle puts there.
template <int R, int BK, int NWAVES, bool ASM = false>
__device__ __forceinline__ void dma_kr(bf16* lds, const bf16* __restrict__ src, int64_t ld, int col0, int ncols,
                                       int k0, int K) {
  constexpr int CPR = R / 8;             // 16-byte chunks per row
  constexpr int TOTAL = BK * CPR;        // chunks per tile
  static_assert(TOTAL % 64 == 0, "whole instructions");
  constexpr int INSTR = TOTAL / 64;
  constexpr bool EVEN = INSTR % NWAVES == 0;
  constexpr int IPW = (INSTR + NWAVES - 1) / NWAVES;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int ins = EVEN ? wave * IPW + i : wave + i * NWAVES;
    if (!EVEN && ins >= INSTR) break;
    const int g = ins * 64 + lane;
    const int k = g / CPR;
    const int c = kr_chunk<R>(k, g % CPR);
    const int gk = k0 + k, gc = col0 + 8 * c;
    const bf16* gp = (gk < K && gc < ncols) ? src + (int64_t)gk * ld + gc : reinterpret_cast<const bf16*>(g2_zero16);
    if constexpr (ASM) dma16_ptr(gp, lds_addr(lds + ins * 512));
    else __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gp), lds + ins * 512, 16, 0, 0);
  }
}

// ---- DMA with per-lane offsets computed once per tile.  For a K step that
// lies wholly inside the matrix, a lane's source address is a uniform base
// (matrix, tile origin and K step: scalar registers) plus a 32-bit byte
// offset fixed for the whole tile, so each wave instruction costs one M0
// write and the load itself.  Rows (K-major) or columns (K-slow) past the
// matrix edge are clamped to the last valid one: they only feed output rows
// or columns that are never stored.  The caller uses dma_rows / dma_kr (zero
// fill) for a ragged last K step.
template <int ROWS, int BK, int NWAVES>
struct RowsDma {
  static constexpr int CPR = BK / 8, RPI = 64 / CPR, INSTR = ROWS / RPI;
  static constexpr bool EVEN = INSTR % NWAVES == 0;
  static constexpr int IPW = (INSTR + NWAVES - 1) / NWAVES;
  static_assert(ROWS % RPI == 0, "whole instructions");
  uint32_t off[IPW];
  int ins0;
  // instruction i of this wave (EVEN: a contiguous run; else dealt in turn)
  __device__ __forceinline__ int ins(int i) const { return EVEN ? ins0 + i : ins0 + i * NWAVES; }
  // tile rows row0 .. row0+ROWS of a [nrows][ld] matrix (row0 < nrows)
  __device__ __forceinline__ void init(int64_t ld, int row0, int nrows) {
    const int lane = threadIdx.x & 63;
    ins0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * (EVEN ? IPW : 1);
    const int last = nrows - 1 - row0;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = min(ins(i), INSTR - 1) * RPI + lane / CPR;
      const int c = swz_chunk<BK>(r, lane % CPR);
      off[i] = (uint32_t)(((int64_t)min(r, last) * ld + 8 * c) * 2);
    }
  }
  // The SwiGLU row map: tile row r stands for virtual column v = row0 + r
  // of a product whose 64-column groups pair gate and up rows of a stacked
  // [2F][ld] matrix (F = nvirt / 2): v = 64 b + w reads row 32 b + w for
  // w < 32 and F + 32 b + w - 32 otherwise.  Offsets are absolute (issue
  // with row0 = 0); rows past nvirt are clamped to the last one.
  __device__ __forceinline__ void init_swiglu(int64_t ld, int row0, int nvirt) {
    const int lane = threadIdx.x & 63;
    ins0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * (EVEN ? IPW : 1);
    const int F = nvirt >> 1;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = min(ins(i), INSTR - 1) * RPI + lane / CPR;
      const int c = swz_chunk<BK>(r, lane % CPR);
      const int v = min(row0 + r, nvirt - 1);
      const int w = v & 63, f = ((v >> 6) << 5) + (w & 31);
      const int row = w < 32 ? f : F + f;
      off[i] = (uint32_t)(((int64_t)row * ld + 8 * c) * 2);
    }
  }
  __device__ __forceinline__ void issue(bf16* lds, const bf16* src, int64_t ld, int row0, int k0) const {
    const char* base = reinterpret_cast<const char*>(src + (int64_t)row0 * ld + k0);
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      if (EVEN || ins(i) < INSTR) dma16_off(base, off[i], lds_addr(lds + ins(i) * RPI * BK));
  }
};

template <int R, int BK, int NWAVES>
struct KrDma {
  static constexpr int CPR = R / 8, TOTAL = BK * CPR, INSTR = TOTAL / 64;
  static constexpr bool EVEN = INSTR % NWAVES == 0;
  static constexpr int IPW = (INSTR + NWAVES - 1) / NWAVES;
  static_assert(TOTAL % 64 == 0, "whole instructions");
  uint32_t off[IPW];
  int ins0;
  __device__ __forceinline__ int ins(int i) const { return EVEN ? ins0 + i : ins0 + i * NWAVES; }
  // tile columns col0 .. col0+R of a [K][ld] matrix (col0 < ncols, ncols % 8 == 0)
  __device__ __forceinline__ void init(int64_t ld, int col0, int ncols) {
    const int lane = threadIdx.x & 63;
    ins0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * (EVEN ? IPW : 1);
    const int last = ncols - 8 - col0;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int g = min(ins(i), INSTR - 1) * 64 + lane;
      const int k = g / CPR;
      const int c = kr_chunk<R>(k, g % CPR);
      off[i] = (uint32_t)(((int64_t)k * ld + min(8 * c, last)) * 2);
    }
  }
  __device__ __forceinline__ void issue(bf16* lds, const bf16* src, int64_t ld, int col0, int k0) const {
    const char* base = reinterpret_cast<const char*>(src + (int64_t)k0 * ld + col0);
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      if (EVEN || ins(i) < INSTR) dma16_off(base, off[i], lds_addr(lds + ins(i) * 512));
  }
};

// Column read of a [rows][R] kr-swizzled tile: this lane gets column
// c0 + (lane % 16) of rows r0 .. r0+3 (r0 % 4 == 0, c0 % 16 == 0).
template <int R>
__device__ __forceinline__ bf16x4 tr_read4_kr(const bf16* tile, int r0, int c0) {
  const int j = threadIdx.x & 15;
  const int row = r0 + (j >> 2);
  const int col = c0 + 4 * (j & 3);
  const int byte = row * (2 * R) + (kr_chunk<R>(row, col >> 3) << 4) + ((col & 7) << 1);
  auto base = (__attribute__((address_space(3))) char*)(tile);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + byte));
  return __builtin_bit_cast(bf16x4, v);
}

}  // namespace g2
