// fa_tile.h -- LDS staging of [rows][D] bf16 tiles for the gfx950 kernels.
//
// Tiles are copied from global memory straight into LDS with global_load_lds_dwordx4
// (no registers in between): one instruction moves 16 bytes per lane and writes lane
// l's bytes at LDS address m0 + 16 l, so each wave-instruction fills 1 KB of LDS
// contiguously. Rows are therefore stored unpadded (D * 2 bytes), and bank conflicts
// are avoided by XOR-swizzling the 16-byte chunks of each row: logical chunk c of row
// r lives at physical chunk c ^ swz(r), swz(r) = ((r & 3) << 2) | ((r >> 2) & 3)
// (reduced modulo the chunks per row). With it, the two read patterns the kernels use
// touch distinct chunks within each LDS phase:
//   * 16-byte row reads by 16 lanes of 16 consecutive rows at one logical chunk
//     (swz is a bijection on 16 consecutive rows);
//   * transpose reads (ds_read_b64_tr_b16) by a 16-lane group of 4 consecutive rows
//     times 16 columns (swz >> 2 differs across the 4 rows).
#pragma once

#include "fa_device.h"

namespace fa {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int D>
struct Tile {
  static constexpr int NCH = D / 8;  // 16-byte chunks per row

  __device__ static __forceinline__ int swz(int row) { return (((row & 3) << 2) | ((row >> 2) & 3)) & (NCH - 1); }

  // element offset of logical 8-element chunk c of row `row`
  __device__ static __forceinline__ int chunk(int row, int c) { return row * D + 8 * (c ^ swz(row)); }

  // element offset of the 4 elements at column col (a multiple of 4) of row `row`
  __device__ static __forceinline__ int quad(int row, int col) { return chunk(row, col >> 3) + (col & 4); }

  // 16-byte read of logical chunk c of row `row`
  __device__ static __forceinline__ bf16x8 read_chunk(const bf16* lds, int row, int c) {
    return *reinterpret_cast<const bf16x8*>(lds + chunk(row, c));
  }

  // transpose read: with lane L of each 16-lane group addressing row r0 + L / 4 at
  // column c0 + 4 (L % 4), lane i receives column c0 + i of rows r0 .. r0 + 3
  __device__ static __forceinline__ bf16x4 read_tr(const bf16* lds, int row, int col) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)((__attribute__((address_space(3))) bf16*)lds + quad(row, col)));
  }

  // Stage rows [0, ROWS) of a tile whose row i is at src + i * stride (elements), rows
  // at or beyond `valid` replaced by row valid - 1 (the callers mask those rows out).
  // NT threads, NT / 64 waves; every thread issues ROWS * NCH / NT loads. The caller
  // waits (vmcnt) and synchronises before reading the tile. A full tile (valid >= ROWS,
  // the common case) costs no vector ALU work per load: a thread loads the same chunk of
  // every row it touches (its loads are RSTEP rows apart and the swizzle repeats every 16
  // rows), so one 32-bit byte offset serves all of them and the row step goes into the
  // scalar base address. The row stride is below 2^24 elements (checked on the host).
  // FAST_FULL = false keeps the per-lane addressing for every tile (the backward's walks,
  // measured faster that way).
  template <int ROWS, int NT, bool FAST_FULL = true>
  __device__ static __forceinline__ void stage(bf16* lds, const bf16* src, int64_t stride, int valid,
                                               int group_wave = -1) {
    constexpr int W = NT / 64, PER = ROWS * NCH / NT, RSTEP = 64 * W / NCH;
    static_assert((ROWS * NCH) % NT == 0, "tile must split evenly over the threads");
    static_assert(!FAST_FULL || RSTEP % 16 == 0, "a thread's rows must share their swizzle");
    // group_wave: this wave's index among the NT / 64 staging waves (default: its index
    // in the workgroup)
    const int lane = threadIdx.x & 63, wave = group_wave < 0 ? (int)(threadIdx.x >> 6) : group_wave;
    if (FAST_FULL && valid >= ROWS) {
      const int row0 = (64 * wave + lane) / NCH;
      const int c = (lane % NCH) ^ swz(row0);
      const uint32_t voff = ((uint32_t)row0 * (uint32_t)stride + 8u * (uint32_t)c) * 2u;
      #pragma unroll
      for (int i = 0; i < PER; ++i)
        dma16(src + (int64_t)RSTEP * i * stride, voff, lds + 8 * 64 * (__builtin_amdgcn_readfirstlane(wave) + W * i));
      return;
    }
    #pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int n0 = 64 * (wave + W * i);  // first chunk of this wave-instruction
      const int n = n0 + lane;
      const int row = n / NCH, p = n % NCH;
      const int c = p ^ swz(row);
      const int grow = row < valid ? row : valid - 1;
      dma16(src + (int64_t)grow * stride + 8 * c, lds + 8 * n0);
    }
  }

  // One wave-instruction of global_load_lds_dwordx4: lane l's 16 bytes from g land at
  // LDS byte address m0 + 16 l, m0 = dst (wave-uniform). Written as asm so that the
  // compiler does not treat the asynchronous LDS write as possibly aliasing every later
  // LDS read (it would wait for the load before the current tile's reads, serialising
  // the prefetch); the callers order the loads with an explicit wait and barrier.
  __device__ static __forceinline__ void dma16(const bf16* g, bf16* dst) {
    const uint32_t m0 =
        __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) bf16*)dst);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0)
                 : "memory", "m0");
  }
  // the same with a wave-uniform base address and a per-lane 32-bit byte offset
  __device__ static __forceinline__ void dma16(const bf16* sbase, uint32_t voff, bf16* dst) {
    const uint32_t m0 =
        __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) bf16*)dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
  }
};

// wait for this wave's outstanding global loads (including loads into LDS)
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace fa
