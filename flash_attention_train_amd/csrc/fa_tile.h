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

#include <type_traits>

#include "fa_device.h"

namespace fa {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A raw buffer resource (stride 0, no swizzle) over the `bytes` bytes at `base`. The range
// check of a load through it covers the scalar and the per-lane offset together: a lane
// whose offset is `bytes` or more reads no memory and returns zeros (for a load into LDS,
// zeros are written there). The fourth word is the gfx9 data-format default that raw loads
// use.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

template <int D>
struct Tile {
  static constexpr int NCH = D / 8;  // 16-byte chunks per row

  __host__ __device__ static __forceinline__ int swz(int row) { return (((row & 3) << 2) | ((row >> 2) & 3)) & (NCH - 1); }

  // element offset of logical 8-element chunk c of row `row`
  __host__ __device__ static __forceinline__ int chunk(int row, int c) { return row * D + 8 * (c ^ swz(row)); }

  // element offset of the 4 elements at column col (a multiple of 4) of row `row`
  __host__ __device__ static __forceinline__ int quad(int row, int col) { return chunk(row, col >> 3) + (col & 4); }

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

  // Stage rows [0, ROWS) of a tile whose row i starts at src + i * stride (elements); rows
  // at or beyond `valid` arrive as zeros. The loads go through a buffer resource that ends
  // after row valid - 1, whose range check turns every later row into zeros without a
  // memory access, so the last tile needs no clamping. A thread loads the same chunk of
  // every row it touches (RSTEP rows apart; the swizzle repeats every 16 rows): one per-lane
  // byte offset serves all its loads and the row step is the scalar offset, so a load costs
  // no vector work. The row stride is below 2^24 elements (checked on the host): the
  // offsets within a tile fit in 32 bits.
  // NT threads (NT / 64 waves) stage the tile; group_wave is this wave's index among them
  // (default: its index in the workgroup). `lds` is the tile's LDS byte address.
  template <int ROWS, int NT>
  __device__ static __forceinline__ void stage_rows(uint32_t lds, const bf16* src, int64_t stride, int valid,
                                                    int group_wave = -1) {
    constexpr int W = NT / 64, PER = ROWS * NCH / NT, RSTEP = 64 * W / NCH;
    static_assert((ROWS * NCH) % NT == 0, "tile must split evenly over the threads");
    const int lane = threadIdx.x & 63;
    const int gw = group_wave < 0 ? (int)(threadIdx.x >> 6) : group_wave;
    const int wave = __builtin_amdgcn_readfirstlane(gw);  // (for the LDS destinations)
    const uint32_t st = (uint32_t)stride;
    const int row0 = (64 * gw + lane) / NCH;
    const int v = valid < ROWS ? valid : ROWS;
    const u32x4 rsrc = raw_rsrc(src, v > 0 ? ((uint32_t)(v - 1) * st + (uint32_t)D) * 2u : 0u);
    if constexpr (RSTEP % 16 == 0) {
      const uint32_t voff = ((uint32_t)row0 * st + 8u * (uint32_t)((lane % NCH) ^ swz(row0))) * 2u;
      #pragma unroll
      for (int i = 0; i < PER; ++i)
        dma16(rsrc, voff, (uint32_t)(RSTEP * i) * st * 2u, lds + 1024u * (uint32_t)(wave + W * i));
    } else {  // (fewer staging waves: a thread's rows differ in their swizzle, one offset each)
      #pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int row = row0 + RSTEP * i;
        const uint32_t voff = ((uint32_t)row * st + 8u * (uint32_t)((lane % NCH) ^ swz(row))) * 2u;
        dma16(rsrc, voff, 0u, lds + 1024u * (uint32_t)(wave + W * i));
      }
    }
  }
  template <int ROWS, int NT>
  __device__ static __forceinline__ void stage_rows(bf16* lds, const bf16* src, int64_t stride, int valid,
                                                    int group_wave = -1) {
    stage_rows<ROWS, NT>(lds_addr(lds), src, stride, valid, group_wave);
  }

  // the LDS byte address of a pointer into LDS: a flat address into LDS is the shared
  // aperture's base, whose low 32 bits are zero, plus the LDS address, so its low word is
  // the LDS address (with no null check to emit)
  __device__ static __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

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
  // the same through a buffer resource: lane l's 16 bytes at byte offset soff + voff (zeros
  // where that is past the resource's end)
  // (dst: the LDS byte address, wave-uniform)
  __device__ static __forceinline__ void dma16(const u32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(m0), "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
  }
  // the same with the non-temporal hint, for data read once (it then displaces less of what
  // the caches hold for later work)
  __device__ static __forceinline__ void dma16nt(const u32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen nt lds" ::"v"(voff), "s"(rsrc),
                 "s"(m0), "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
  }
};

// ---------------------------------------------------------------------------
// K / V stored as fp16 or q8_0, read in place: 8 consecutive values of a row to bf16
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// fp16 -> bf16: the fp32 widening is exact; one rounding to nearest even
__device__ __forceinline__ bf16x8 cvt8_f16(const f16x8& h) {
  bf16x8 o;
  #pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = (bf16)(float)h[j];
  return o;
}
// q8_0 -> bf16: value = d * q, the fp32 product of an fp16 scale and an int8 quant is exact
// (at most 11 + 7 significant bits); one rounding to nearest even
__device__ __forceinline__ bf16x8 cvt8_q8(uint2 q, _Float16 d) {
  const float df = (float)d;
  bf16x8 o;
  #pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = j < 4 ? q.x : q.y;
    const int v = __builtin_amdgcn_sbfe((int)w, 8 * (j & 3), 8);
    o[j] = (bf16)((float)v * df);
  }
  return o;
}
// 8 values of a stored row (element j0 .. j0 + 7, j0 a multiple of 8) as bf16: `row` points at
// the row's first stored element (fp16 or int8), `srow` at its first q8_0 scale
template <int KVF>
__device__ __forceinline__ bf16x8 load_cvt8(const void* row, const _Float16* srow, int j0) {
  if constexpr (KVF == 1) {
    return cvt8_f16(*reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(row) + j0));
  } else {
    return cvt8_q8(*reinterpret_cast<const uint2*>(static_cast<const int8_t*>(row) + j0), srow[j0 >> 5]);
  }
}

// A [ROWS][D] K or V tile stored as fp16 (KVF 1) or q8_0 (KVF 2), staged into LDS in the
// same swizzled bf16 layout as Tile<D>::stage: load() issues this thread's global loads
// (row `valid - 1` repeated past the end), commit() converts them and writes LDS. Between
// the two the raw values wait in registers, so the loads of the next tile can be issued
// before the current tile's products and written after them.
template <int D, int ROWS, int NT, int KVF>
struct CvtStage {
  static constexpr int NCH = D / 8, W = NT / 64, PER = ROWS * NCH / NT;
  static_assert((ROWS * NCH) % NT == 0, "tile must split evenly over the threads");
  typedef typename std::conditional<KVF == 1, f16x8, uint2>::type Raw;
  Raw raw[PER];
  _Float16 sc[PER];
  __device__ __forceinline__ void load(const void* src, int64_t stride, const _Float16* scale, int64_t sstride,
                                       int valid, int group_wave = -1) {
    const int lane = threadIdx.x & 63, wave = group_wave < 0 ? (int)(threadIdx.x >> 6) : group_wave;
    #pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int n = 64 * (wave + W * i) + lane;
      const int row = n / NCH, p = n % NCH;
      const int c = p ^ Tile<D>::swz(row);
      const int64_t grow = row < valid ? row : valid - 1;
      if constexpr (KVF == 1) {
        raw[i] = *reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(src) + grow * stride + 8 * c);
      } else {
        raw[i] = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(src) + grow * stride + 8 * c);
        sc[i] = scale[grow * sstride + (c >> 2)];
      }
    }
  }
  __device__ __forceinline__ void commit(bf16* lds, int group_wave = -1) const {
    const int lane = threadIdx.x & 63, wave = group_wave < 0 ? (int)(threadIdx.x >> 6) : group_wave;
    #pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int n = 64 * (wave + W * i) + lane;
      bf16x8 v;
      if constexpr (KVF == 1) v = cvt8_f16(raw[i]);
      else v = cvt8_q8(raw[i], sc[i]);
      *reinterpret_cast<bf16x8*>(lds + 8 * n) = v;
    }
  }
};

// wait for this wave's outstanding global loads (including loads into LDS)
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0); }

// s_waitcnt operand (gfx9 encoding) that waits until at most n vector memory instructions of
// this wave are outstanding, and for nothing else. Loads complete in issue order, so waiting
// down to n leaves exactly the n most recent ones in flight (no stores may be among those
// counted).
constexpr int vmcnt_enc(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

}  // namespace fa
