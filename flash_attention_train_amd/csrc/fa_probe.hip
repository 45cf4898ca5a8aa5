// fa_probe.hip -- layout probes for the matrix-core and LDS-transpose
// instructions (include/fa_train_probe.h). Test support: each wave executes one
// instruction on register contents chosen by the caller and returns its raw
// per-lane result, so the lane maps used by the kernels can be derived and
// asserted instead of assumed ("Flash Attn Training" skill page, section 6,
// trap 10: an operand's lane map need not equal the accumulator's).
#include "fa_device.h"
#include "fa_train_probe.h"

namespace {

using namespace fa;

typedef short short4_t __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(64) void mfma_probe_kernel(const float* a, const float* b, float* c) {
  const int w = blockIdx.x, l = threadIdx.x;
  if (KIND == FA_PROBE_MFMA_32X32X16_BF16 || KIND == FA_PROBE_MFMA_16X16X32_BF16) {
    bf16x8 av, bv;
    for (int j = 0; j < 8; ++j) {
      av[j] = (bf16)a[((int64_t)w * 64 + l) * 8 + j];
      bv[j] = (bf16)b[((int64_t)w * 64 + l) * 8 + j];
    }
    if (KIND == FA_PROBE_MFMA_32X32X16_BF16) {
      f32x16 acc;
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
      for (int r = 0; r < 16; ++r) c[((int64_t)w * 64 + l) * 16 + r] = acc[r];
    } else {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
      for (int r = 0; r < 4; ++r) c[((int64_t)w * 64 + l) * 4 + r] = acc[r];
    }
  } else {
    const float av = a[(int64_t)w * 64 + l], bv = b[(int64_t)w * 64 + l];
    if (KIND == FA_PROBE_MFMA_32X32X2_F32) {
      f32x16 acc;
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
      for (int r = 0; r < 16; ++r) c[((int64_t)w * 64 + l) * 16 + r] = acc[r];
    } else {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
      for (int r = 0; r < 4; ++r) c[((int64_t)w * 64 + l) * 4 + r] = acc[r];
    }
  }
}

__global__ __launch_bounds__(64) void tr16_probe_kernel(const int32_t* addr, uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4096];
  const int w = blockIdx.x, l = threadIdx.x;
  for (int i = l; i < 4096; i += 64) lds[i] = (uint16_t)i;
  __syncthreads();
  const int raw = addr[(int64_t)w * 64 + l];
  const bool ok = raw >= 0 && raw <= 8184 && (raw % 8) == 0;  // in-bounds, 8-byte aligned
  const int byte = ok ? raw : 0;
  typedef __attribute__((address_space(3))) short4_t lds_short4;
  lds_short4* p = (lds_short4*)((__attribute__((address_space(3))) char*)((__attribute__((address_space(3))) uint16_t*)lds) + byte);
  short4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
  if (!ok) r = short4_t{-1, -1, -1, -1};
  for (int j = 0; j < 4; ++j) out[((int64_t)w * 64 + l) * 4 + j] = (uint16_t)r[j];
}

}  // namespace

extern "C" fa_status fa_train_probe_mfma(int32_t kind, int32_t waves, const float* a, const float* b, float* c,
                                         hipStream_t stream) {
  if (!a || !b || !c) return FA_ERR_NULL;
  if (waves < 1 || waves > 65536) return FA_ERR_SHAPE;
  switch (kind) {
    case FA_PROBE_MFMA_32X32X16_BF16:
      hipLaunchKernelGGL(mfma_probe_kernel<FA_PROBE_MFMA_32X32X16_BF16>, dim3(waves), dim3(64), 0, stream, a, b, c);
      break;
    case FA_PROBE_MFMA_16X16X32_BF16:
      hipLaunchKernelGGL(mfma_probe_kernel<FA_PROBE_MFMA_16X16X32_BF16>, dim3(waves), dim3(64), 0, stream, a, b, c);
      break;
    case FA_PROBE_MFMA_32X32X2_F32:
      hipLaunchKernelGGL(mfma_probe_kernel<FA_PROBE_MFMA_32X32X2_F32>, dim3(waves), dim3(64), 0, stream, a, b, c);
      break;
    case FA_PROBE_MFMA_16X16X4_F32:
      hipLaunchKernelGGL(mfma_probe_kernel<FA_PROBE_MFMA_16X16X4_F32>, dim3(waves), dim3(64), 0, stream, a, b, c);
      break;
    default:
      return FA_ERR_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" fa_status fa_train_probe_ds_read_tr16(int32_t waves, const int32_t* byte_addr, uint16_t* out,
                                                 hipStream_t stream) {
  // Addresses are device-side; the kernel replaces any address outside [0, 8184] or
  // not a multiple of 8 by 0 and reports 0xFFFF for that lane.
  if (!byte_addr || !out) return FA_ERR_NULL;
  if (waves < 1 || waves > 4096) return FA_ERR_SHAPE;
  hipLaunchKernelGGL(tr16_probe_kernel, dim3(waves), dim3(64), 0, stream, byte_addr, out);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
