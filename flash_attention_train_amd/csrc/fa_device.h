// fa_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core conventions (32x32 family, wave64), as asserted by the layout probe
// test:
//   A operand (M x K): lane l holds row m = l % 32; its register slot j (of 8)
//                      carries k-slot (l / 32, j).
//   B operand (K x N): lane l holds column n = l % 32; register slot j carries the
//                      same k-slot (l / 32, j).
//   accumulator (M x N, 16 fp32 registers): lane l, register r holds
//                      n = l % 32, m = 8 * (r / 4) + 4 * (l / 32) + r % 4.
// Only the pairing of k-slots between A and B matters for a product, so a kernel
// may assign any concrete index to k-slot (g, j) as long as both operands agree.
// For bf16 one v_mfma_f32_32x32x16_bf16 consumes all 8 slots; for fp32 eight
// v_mfma_f32_32x32x2_f32 consume slot j each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct f32x8 {
  f32x4 lo, hi;
};

template <typename T>
struct FragT;
template <>
struct FragT<bf16> {
  typedef bf16x8 type;
};
template <>
struct FragT<float> {
  typedef f32x8 type;
};
template <typename T>
using Frag = typename FragT<T>::type;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// matrix-core products: acc += A * B over one 16-long k-slot group
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mma(f32x16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// acc += a b with the accumulator in AGPRs (sums that live there for a whole walk, which
// leaves the arch VGPRs to the operands in flight). The s_nop gives the two wait states
// a VALU write of a source operand needs before a matrix product.
__device__ __forceinline__ void mma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// the last products into AGPR accumulators must have written them before VALU reads
// them (the matrix core's result latency, with margin)
template <int N>
__device__ __forceinline__ void settle_acc(f32x16 (&acc)[N]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
  #pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(acc[i]));
}
__device__ __forceinline__ void mma(f32x16& c, const f32x8& a, const f32x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[3], b.hi[3], c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// fragment loads (8 consecutive elements, or two runs of 4) and conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ void zero(bf16x8& f) {
  #pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)0.0f;
}
__device__ __forceinline__ void zero(f32x8& f) {
  f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
  f.hi = f32x4{0.f, 0.f, 0.f, 0.f};
}

// 8 contiguous elements (16-byte aligned for bf16, 16-byte aligned halves for fp32)
__device__ __forceinline__ void load8(bf16x8& f, const bf16* p) { f = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void load8(f32x8& f, const float* p) {
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void store8(bf16* p, const bf16x8& f) { *reinterpret_cast<bf16x8*>(p) = f; }
__device__ __forceinline__ void store8(float* p, const f32x8& f) {
  *reinterpret_cast<f32x4*>(p) = f.lo;
  *reinterpret_cast<f32x4*>(p + 4) = f.hi;
}

// two runs of 4 contiguous elements (8-byte aligned for bf16, 16-byte for fp32)
__device__ __forceinline__ void load4x2(bf16x8& f, const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  f = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void load4x2(f32x8& f, const float* p0, const float* p1) {
  f.lo = *reinterpret_cast<const f32x4*>(p0);
  f.hi = *reinterpret_cast<const f32x4*>(p1);
}

__device__ __forceinline__ float elem(const bf16x8& f, int j) { return (float)f[j]; }
__device__ __forceinline__ float elem(const f32x8& f, int j) { return j < 4 ? f.lo[j] : f.hi[j - 4]; }

// 8 fp32 values (register slots r0 .. r0 + 7 of an accumulator) to an operand fragment
__device__ __forceinline__ void pack8(bf16x8& f, const f32x16& c, int r0) {
  #pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)c[r0 + j];
}
__device__ __forceinline__ void pack8(f32x8& f, const f32x16& c, int r0) {
  f.lo = f32x4{c[r0 + 0], c[r0 + 1], c[r0 + 2], c[r0 + 3]};
  f.hi = f32x4{c[r0 + 4], c[r0 + 5], c[r0 + 6], c[r0 + 7]};
}

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return (bf16)x;
}
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x combined with the value of the lane 32 positions away (the other half of the wave),
// the same result in both lanes: one v_permlane32_swap of x with itself leaves the lower
// half's values in one register and the upper half's in the other, across the whole wave
// (no LDS round trip)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// x where bit `bit` of `word` is set, -inf where it is clear: a sign-extended one-bit
// field selects between x and -inf bitwise (v_bfe_i32 + v_bitop3, no compare)
__device__ __forceinline__ float ninf_unless_bit(float x, uint32_t word, int bit) {
  const int m = __builtin_amdgcn_sbfe((int)word, bit, 1);
  return __int_as_float((__float_as_int(x) & m) | (~m & (int)0xff800000u));
}

// bits [lo, hi) of a 64-bit word set (0 <= lo, hi <= 64)
__device__ __forceinline__ uint64_t bit_range64(int lo, int hi) {
  const uint64_t below_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
  const uint64_t from_lo = lo >= 64 ? 0ull : (~0ull << lo);
  return below_hi & from_lo;
}

}  // namespace fa
