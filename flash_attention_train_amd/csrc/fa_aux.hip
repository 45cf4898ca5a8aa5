// fa_aux.hip -- the memory-bound helpers of the backward:
//   * the preprocess Delta_i = sum_d dO_id * O_id (llama.cpp pull request 57,
//     commit 86c140d: the tiled backward computes the LSE, then D, then the
//     gradients per tile);
//   * clearing the fp32 dQ accumulator;
//   * converting the accumulated dQ to its output dtype with the softmax scale;
//   * classifying the additive mask's 64 x 64 blocks for the forward and backward;
//   * the gradient of the attention sinks from the LSE and Delta;
//   * the bf16 values of a q8_0-stored K/V window.
// The first three stream their operands once with 16-byte loads and stores.
#include <algorithm>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

// One query row per D/8 consecutive lanes, 8 elements per lane, fp32 products, reduced with
// lane shuffles inside the row's lane group. A workgroup takes kPreRows rows of one (batch,
// head), each thread kPreRows / (256 / (D / 8)) of them with all their loads in flight.
constexpr int kPreRows = 64;
template <typename T, int D>
__global__ __launch_bounds__(256) void preprocess_kernel(const PreArgs p) {
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPB = 256 / LPR;          // rows per pass of the workgroup
  constexpr int RPT = kPreRows / RPB;     // rows per thread
  const int sub = threadIdx.x % LPR;
  const int h = blockIdx.y, b = blockIdx.z;
  const int i0 = blockIdx.x * kPreRows + threadIdx.x / LPR;
  const T* O = static_cast<const T*>(p.o) + b * p.so.b + h * p.so.h + 8 * sub;
  const T* dO = static_cast<const T*>(p.dout) + b * p.sdo.b + h * p.sdo.h + 8 * sub;
  Frag<T> o[RPT], d[RPT];
  #pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int i = i0 + j * RPB;
    if (i < p.Sq) {
      load8(o[j], O + (int64_t)i * p.so.s);
      load8(d[j], dO + (int64_t)i * p.sdo.s);
    } else {
      zero(o[j]);
      zero(d[j]);
    }
  }
  float acc[RPT];
  #pragma unroll
  for (int j = 0; j < RPT; ++j) {
    acc[j] = 0.f;
    for (int e = 0; e < 8; ++e) acc[j] += elem(o[j], e) * elem(d[j], e);
  }
  #pragma unroll
  for (int j = 0; j < RPT; ++j)
    for (int off = LPR / 2; off > 0; off >>= 1) acc[j] += __shfl_xor(acc[j], off, 64);
  if (sub == 0) {
    float* delta = p.delta + b * p.delta_sb + h * p.delta_sh;
    #pragma unroll
    for (int j = 0; j < RPT; ++j)
      if (i0 + j * RPB < p.Sq) delta[i0 + j * RPB] = acc[j];
  }
}

__global__ __launch_bounds__(256) void zero_kernel(f32x4* p, int64_t n4) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) p[i] = z;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void dq_convert_kernel(const DqArgs p) {
  constexpr int CPR = D / 8;  // 8-element chunks per row
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nrows = (int64_t)p.B * p.Hq * p.Sq;
  if (c >= nrows * CPR) return;
  const int64_t row = c / CPR;
  const int d0 = (int)(c % CPR) * 8;
  const int i = (int)(row % p.Sq);
  const int h = (int)((row / p.Sq) % p.Hq);
  const int b = (int)(row / ((int64_t)p.Sq * p.Hq));
  const float* src = p.dq_acc + row * D + d0;
  const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
  T* dst = static_cast<T*>(p.dq) + b * p.sdq.b + h * p.sdq.h + (int64_t)i * p.sdq.s + d0;
  Frag<T> out;
  f32x16 tmp;
  for (int j = 0; j < 4; ++j) {
    tmp[j] = lo[j] * p.scale;
    tmp[4 + j] = hi[j] * p.scale;
  }
  pack8(out, tmp, 0);
  store8(dst, out);
}

// Sum of the backward's fp32 partial slices, 8 consecutive elements per thread: each
// slice element is read once, the result written once (or added to an fp32 output). A
// workgroup takes 256 / (D / 8) rows of one (batch, head) of one of up to three tensors.
template <typename T, int D>
__global__ __launch_bounds__(256) void reduce_parts_kernel(const ReduceArgs p0, const ReduceArgs p1,
                                                           const ReduceArgs p2, const int ntiles) {
  // one launch reduces up to three tensors of one output dtype (dK, dV and dQ): grid
  // (batch entries x ntiles row tiles, heads, tensors)
  const int b = blockIdx.x / ntiles, tile = blockIdx.x % ntiles, h = blockIdx.y;
  const ReduceArgs& p = blockIdx.z == 0 ? p0 : blockIdx.z == 1 ? p1 : p2;
  constexpr int CPR = D / 8;
  if (b >= p.B || h >= p.H) return;
  const int i = tile * (256 / CPR) + threadIdx.x / CPR;
  if (i >= p.S) return;
  const int d0 = (threadIdx.x % CPR) * 8;
  const float* src = p.parts + (((int64_t)b * p.H + h) * p.S_parts + i) * D + d0;
  f32x16 acc;
  #pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  #pragma unroll 4
  for (int s = 0; s < p.nparts; ++s) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(src + s * p.part_stride);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(src + s * p.part_stride + 4);
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += lo[j];
      acc[4 + j] += hi[j];
    }
  }
  T* dst = static_cast<T*>(p.out) + b * p.so.b + h * p.so.h + (int64_t)i * p.so.s + d0;
  if (p.accumulate) {  // fp32 output only (checked by the caller)
    float* f = reinterpret_cast<float*>(dst);
    #pragma unroll
    for (int j = 0; j < 8; ++j) f[j] += acc[j] * p.scale;
    return;
  }
  #pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] *= p.scale;
  Frag<T> out;
  pack8(out, acc, 0);
  store8(dst, out);
}

// One workgroup per 64 x 64 mask block (clipped at Sq and Sk; entries outside count as
// masked for the bits and are ignored by the class). Each wave takes 16 consecutive
// rows with all 16 loads in flight at once; a wave ballot per row gives the row word,
// a 64 x 64 bit transpose across the lanes of wave 0 (six butterfly rounds of lane
// exchanges) gives the column words, and the class comes from OR-ed flags.
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m) {
  const int lo = __shfl_xor((int)(uint32_t)x, m, 64), hi = __shfl_xor((int)(uint32_t)(x >> 32), m, 64);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__global__ __launch_bounds__(256) void mask_tiles_kernel(const AttnShape a, uint8_t* tiles, uint64_t* rowbits,
                                                         uint64_t* colbits) {
  __shared__ uint64_t rows_lds[kMaskTile];
  __shared__ int flags_lds;
  const int ct = blockIdx.x, rt = blockIdx.y, bm = blockIdx.z;
  const int64_t blk = ((int64_t)bm * gridDim.y + rt) * gridDim.x + ct;
  const float* M = a.mask + bm * a.mask_sb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int key = ct * kMaskTile + lane;
  const int row0 = rt * kMaskTile + wave * 16;
  if (threadIdx.x == 0) flags_lds = 0;
  float v[16];
  #pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool in = row0 + i < a.Sq && key < a.Sk;
    v[i] = in ? M[(int64_t)(row0 + i) * a.mask_sq + key] : neg_inf();
  }
  int fl = 0;  // 1: a visible entry, 2: a masked entry inside the block, 4: a nonzero visible value
  #pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool in = row0 + i < a.Sq && key < a.Sk;
    const bool vis = v[i] != neg_inf();
    fl |= (vis ? 1 : 0) | (in && !vis ? 2 : 0) | (vis && v[i] != 0.f ? 4 : 0);
    const uint64_t w = __ballot(vis);
    if (lane == 0) {
      rows_lds[wave * 16 + i] = w;
      rowbits[blk * kMaskTile + wave * 16 + i] = w;
    }
  }
  const int wf = (__any(fl & 1) ? 1 : 0) | (__any(fl & 2) ? 2 : 0) | (__any(fl & 4) ? 4 : 0);
  __syncthreads();  // flags cleared, row words in LDS
  if (lane == 0) atomicOr(&flags_lds, wf);
  if (wave == 0) {
    // lane r holds row r's word (bit c: key c); after the rounds lane c holds column c's
    // word (bit r: row r)
    uint64_t x = rows_lds[lane];
    const uint64_t masks[6] = {0x00000000FFFFFFFFull, 0x0000FFFF0000FFFFull, 0x00FF00FF00FF00FFull,
                               0x0F0F0F0F0F0F0F0Full, 0x3333333333333333ull, 0x5555555555555555ull};
    #pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int j = 32 >> k;
      const uint64_t other = shfl_xor64(x, j);
      if (lane & j)
        x ^= ((other >> j) ^ x) & masks[k];
      else
        x ^= (((x >> j) ^ other) & masks[k]) << j;
    }
    colbits[blk * kMaskTile + lane] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int f = flags_lds;
    tiles[blk] = !(f & 1) ? kTileDead : (f & 4) ? kTileBias : (f & 2) ? kTileBits : kTileOpen;
  }
}

template <typename T, int D>
hipError_t launch_pre_t(const PreArgs& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.Sq + kPreRows - 1) / kPreRows), p.Hq, p.B);
  hipLaunchKernelGGL((preprocess_kernel<T, D>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dq_t(const DqArgs& p, hipStream_t stream) {
  const int64_t chunks = (int64_t)p.B * p.Hq * p.Sq * (D / 8);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  hipLaunchKernelGGL((dq_convert_kernel<T, D>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Gradient of the attention sinks: one workgroup per (chunk of a head's B * Sq rows,
// head); every thread sums exp(sink - LSE) * Delta over its rows, the workgroup reduces
// the sums (lane shuffles, then one value per wave in LDS) and adds the negated total
// to dsink[h] with one atomic.
constexpr int kSinkRows = 2048;  // rows per workgroup
__global__ __launch_bounds__(256) void sink_grad_kernel(const SinkArgs p) {
  const int h = blockIdx.y;
  const int64_t rows = (int64_t)p.B * p.Sq;
  const float sink = p.sinks[h];
  float acc = 0.f;
  for (int64_t r = (int64_t)blockIdx.x * kSinkRows + threadIdx.x; r < min(rows, (int64_t)(blockIdx.x + 1) * kSinkRows);
       r += 256) {
    const int b = (int)(r / p.Sq), i = (int)(r % p.Sq);
    const float lse = p.lse[b * p.lse_sb + h * p.lse_sh + i];
    const float dl = p.delta[b * p.delta_sb + h * p.delta_sh + i];
    acc += expf(sink - lse) * dl;
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(p.dsink + h, -(part[0] + part[1] + part[2] + part[3]));
}

// q8_0 window rows to bf16: one thread per 16 consecutive values of a row (one 16-byte
// load of quants, the block's fp16 scale, two 16-byte stores). The fp32 product of an
// fp16 scale and an int8 quant is exact; the one rounding is to bf16 (nearest even).
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const DequantArgs p) {
  const int per_row = p.D / 16;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  if (t >= rows * per_row) return;
  const int64_t row = t / per_row;
  const int c16 = (int)(t % per_row);
  const int s = (int)(row % p.S), h = (int)((row / p.S) % p.H), b = (int)(row / ((int64_t)p.S * p.H));
  typedef int8_t i8x16 __attribute__((ext_vector_type(16)));
  const i8x16 q = *reinterpret_cast<const i8x16*>(p.qs + b * p.sq.b + h * p.sq.h + (int64_t)s * p.sq.s + 16 * c16);
  const float d = (float)p.d[b * p.sd.b + h * p.sd.h + (int64_t)s * p.sd.s + c16 / 2];
  bf16x8 lo, hi;
  #pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = (bf16)(d * (float)q[e]);
    hi[e] = (bf16)(d * (float)q[8 + e]);
  }
  bf16* o = static_cast<bf16*>(p.out) + b * p.so.b + h * p.so.h + (int64_t)s * p.so.s + 16 * c16;
  *reinterpret_cast<bf16x8*>(o) = lo;
  *reinterpret_cast<bf16x8*>(o + 8) = hi;
}

// f16 window rows to the compute type: one thread per 8 consecutive values of a row (one
// 16-byte load). fp16 -> fp32 is exact (subnormals included); fp16 -> bf16 keeps 8 of the
// 11 significand bits, rounding to nearest even, and loses no range (bf16 spans fp16's).
template <bool TO_BF16>
__global__ __launch_bounds__(256) void convert_f16_kernel(const ConvertArgs p) {
  const int per_row = p.D / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  if (t >= rows * per_row) return;
  const int64_t row = t / per_row;
  const int c8 = (int)(t % per_row);
  const int s = (int)(row % p.S), h = (int)((row / p.S) % p.H), b = (int)(row / ((int64_t)p.S * p.H));
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const f16x8 x = *reinterpret_cast<const f16x8*>(p.src + b * p.ss.b + h * p.ss.h + (int64_t)s * p.ss.s + 8 * c8);
  const int64_t o = b * p.so.b + h * p.so.h + (int64_t)s * p.so.s + 8 * c8;
  if constexpr (TO_BF16) {
    bf16x8 y;
    #pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (bf16)(float)x[e];
    *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.out) + o) = y;
  } else {
    float4 lo, hi;
    lo.x = (float)x[0], lo.y = (float)x[1], lo.z = (float)x[2], lo.w = (float)x[3];
    hi.x = (float)x[4], hi.y = (float)x[5], hi.z = (float)x[6], hi.w = (float)x[7];
    float* y = static_cast<float*>(p.out) + o;
    *reinterpret_cast<float4*>(y) = lo;
    *reinterpret_cast<float4*>(y + 4) = hi;
  }
}

}  // namespace

hipError_t launch_convert_f16(const ConvertArgs& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.B * p.H * p.S * (p.D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (p.to_bf16)
    hipLaunchKernelGGL(convert_f16_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(convert_f16_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_dequant_q8_0(const DequantArgs& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.B * p.H * p.S * (p.D / 16);
  hipLaunchKernelGGL(dequant_q8_0_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_sink_grad(const SinkArgs& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.Sq;
  const dim3 grid((unsigned)((rows + kSinkRows - 1) / kSinkRows), p.Hq);
  hipLaunchKernelGGL(sink_grad_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_preprocess(const PreArgs& p, int is_bf16, hipStream_t stream) {
  if (is_bf16) return p.D == 64 ? launch_pre_t<bf16, 64>(p, stream) : launch_pre_t<bf16, 128>(p, stream);
  return p.D == 64 ? launch_pre_t<float, 64>(p, stream) : launch_pre_t<float, 128>(p, stream);
}

hipError_t launch_mask_tiles(const AttnShape& a, uint8_t* tiles, hipStream_t stream) {
  const int nrt = (a.Sq + kMaskTile - 1) / kMaskTile, nct = (a.Sk + kMaskTile - 1) / kMaskTile;
  const int bm = a.mask_sb == 0 ? 1 : a.B;
  hipLaunchKernelGGL(mask_tiles_kernel, dim3(nct, nrt, bm), dim3(256), 0, stream, a, tiles,
                     const_cast<uint64_t*>(a.rowbits), const_cast<uint64_t*>(a.colbits));
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream) {
  // n is a multiple of 4 (whole rows of D = 64 or 128 floats)
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<f32x4*>(p), n4);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_reduce_t(const ReduceArgs& p, const ReduceArgs* p1, const ReduceArgs* p2, hipStream_t stream) {
  // the grid covers the largest of the tensors; the others' workgroups past their ends return
  // at once
  int S = p.S, H = p.H, B = p.B;
  for (const ReduceArgs* q : {p1, p2})
    if (q) {
      S = std::max(S, q->S);
      H = std::max(H, q->H);
      B = std::max(B, q->B);
    }
  const int rows_per_wg = 256 / (D / 8), n = p2 ? 3 : p1 ? 2 : 1, ntiles = (S + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)((int64_t)ntiles * B), H, n);
  hipLaunchKernelGGL((reduce_parts_kernel<T, D>), grid, dim3(256), 0, stream, p, p1 ? *p1 : p, p2 ? *p2 : p,
                     ntiles);
  return hipGetLastError();
}

hipError_t launch_reduce_parts(const ReduceArgs& p, const ReduceArgs* p1, const ReduceArgs* p2, int is_bf16,
                               hipStream_t stream) {
  if (is_bf16)
    return p.D == 64 ? launch_reduce_t<bf16, 64>(p, p1, p2, stream) : launch_reduce_t<bf16, 128>(p, p1, p2, stream);
  return p.D == 64 ? launch_reduce_t<float, 64>(p, p1, p2, stream) : launch_reduce_t<float, 128>(p, p1, p2, stream);
}

hipError_t launch_dq_convert(const DqArgs& p, int is_bf16, hipStream_t stream) {
  if (is_bf16) return p.D == 64 ? launch_dq_t<bf16, 64>(p, stream) : launch_dq_t<bf16, 128>(p, stream);
  return p.D == 64 ? launch_dq_t<float, 64>(p, stream) : launch_dq_t<float, 128>(p, stream);
}

}  // namespace fa
