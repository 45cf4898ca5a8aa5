// fa_bwd.hip -- backward of the fused attention op: dQ, dK, dV.
//
// The backward recomputes P from the forward's LSE, tile by tile over the KV
// window, and adds the dK/dV of every query head of a group into the group's KV
// head inside the kernel (llama.cpp pull request 57, commit 86c140d, the tiled
// backward; native GQA without head expansion, "Flash Attn Training" skill page,
// section 6, trap 5).
//
// Work split (KV-stationary): one workgroup per (batch, KV head, BN-key tile),
// NW waves of 32 keys each. The workgroup walks every query head of its group and
// every query tile that can see its keys; dK and dV for its keys accumulate in
// registers across the whole walk, so the group sum needs no atomics. Per query
// tile each wave computes, for its 32 keys:
//   S  = Q K^T        (A: Q rows from LDS,  B: K rows in registers)
//   dP = dO V^T       (A: dO rows from LDS, B: V rows in registers)
//   P  = exp2(S c + M log2e - LSE log2e),  dS = P (dP - Delta)
//   (with a logit softcap c': S c becomes c' tanh(S scale / c') log2e, and dS carries
//   the derivative of the cap, 1 - tanh^2)
//   dV += P^T dO      (A: P straight from the accumulator, B: dO^T from LDS)
//   dK += dS^T Q      (A: dS from the accumulator,        B: Q^T from LDS)
// The accumulator layout puts one key and 16 query rows in each lane, which is
// exactly the A operand of the two products over query rows. dS is then staged
// in LDS and the workgroup computes dQ += dS K for the tile over all its BN keys,
// adding the result into an fp32 dQ accumulator with atomics (other key tiles
// add to the same rows).
//
// Masked entries get P = 0 exactly (so dS = 0): a fully masked query row (LSE 0)
// contributes nothing, and a key column no query can see ends with dK = dV = 0
// exactly (skill page, section 6, trap 8). The rows that see a key by the structure
// (sequence end, key and query lengths, causal diagonal, window) come from the range helper
// the bf16 kernels share; ALiBi adds -slope |key - position| after the cap, like the mask;
// an attention sink only enters through the LSE (its own gradient is a separate pass).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

__device__ __forceinline__ f32x16 zeros16() {
  f32x16 z;
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

__device__ __forceinline__ bf16 elem_t(const bf16x8& f, int j) { return f[j]; }
__device__ __forceinline__ float elem_t(const f32x8& f, int j) { return j < 4 ? f.lo[j] : f.hi[j - 4]; }

__device__ __forceinline__ void atomic_add_f32(float* p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int D, int NW, bool MASK>
__global__ __launch_bounds__(NW * 64, 1) void bwd_kernel(const BwdArgs args) {
  constexpr int NT = NW * 64;
  constexpr int BN = 32 * NW;                     // keys per workgroup
  constexpr int BM = sizeof(T) == 2 ? 64 : 32;    // query rows per tile
  constexpr int QB = BM / 32;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int RS = D + PAD;    // Q / dO tiles [BM][D]
  constexpr int TS = BM + PAD;   // Q^T / dO^T tiles [D][BM]
  constexpr int KTS = BN + PAD;  // K^T tile [D][BN]
  constexpr int SS = BN + PAD;   // dS tile [BM][BN]
  constexpr int DS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) T q_lds[BM * RS];
  __shared__ __attribute__((aligned(16))) T do_lds[BM * RS];
  __shared__ __attribute__((aligned(16))) T qt_lds[D * TS];
  __shared__ __attribute__((aligned(16))) T dot_lds[D * TS];
  __shared__ __attribute__((aligned(16))) T kt_lds[D * KTS];
  __shared__ __attribute__((aligned(16))) T ds_lds[BM * SS];
  __shared__ float lse_lds[BM];
  __shared__ float dlt_lds[BM];

  const AttnShape& a = args.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int b = blockIdx.z, hk = blockIdx.y;
  const int n0 = blockIdx.x * BN;
  const int key = n0 + 32 * wave + r32;  // this lane's key in S / dP accumulators
  const float cs = a.scale * kLog2e;
  const bool capped = a.softcap > 0.f;
  const float cap_in = capped ? a.scale / a.softcap : 0.f, cap_out = a.softcap * kLog2e;

  const T* K = static_cast<const T*>(args.k) + b * args.sk.b + hk * args.sk.h;
  const T* V = static_cast<const T*>(args.v) + b * args.sv.b + hk * args.sv.h;

  // K and V rows of this lane's key as B operands (d = 16 s + 8 g + j)
  Frag<T> kf[DS], vf[DS];
  for (int s = 0; s < DS; ++s) {
    if (key < a.Sk) {
      load8(kf[s], K + (int64_t)key * args.sk.s + 16 * s + 8 * g);
      load8(vf[s], V + (int64_t)key * args.sv.s + 16 * s + 8 * g);
    } else {
      zero(kf[s]);
      zero(vf[s]);
    }
  }
  // K^T of the whole key tile, for the dQ product (B operand: column d, keys)
  for (int c = tid; c < BN * D / 8; c += NT) {
    const int kl = c / (D / 8), d0 = (c % (D / 8)) * 8;
    Frag<T> kv;
    if (n0 + kl < a.Sk)
      load8(kv, K + (int64_t)(n0 + kl) * args.sk.s + d0);
    else
      zero(kv);
    for (int i = 0; i < 8; ++i) kt_lds[(d0 + i) * KTS + kl] = elem_t(kv, i);
  }

  f32x16 dk[DB], dv[DB];
  for (int db = 0; db < DB; ++db) {
    dk[db] = zeros16();
    dv[db] = zeros16();
  }

  // the rows this lane's key sees by the structure, and the query tiles any key of the
  // workgroup's tile sees (both ends of a key's row range move down with the key)
  const int klen = klen_of(a, b), qlen = qlen_of(a, b);
  int64_t rlo, rhi;
  row_range(a, klen, qlen, key, rlo, rhi);
  const int nqt = (a.Sq + BM - 1) / BM;
  int qt_begin = 0, qt_end = 0;
  if (n0 < klen) {
    int64_t lo0, hi0, lo1, hi1;
    row_range(a, klen, qlen, n0, lo0, hi0);
    row_range(a, klen, qlen, min(n0 + BN, klen) - 1, lo1, hi1);
    qt_begin = (int)min<int64_t>(lo0 / BM, nqt);
    qt_end = hi1 > lo0 ? (int)min<int64_t>((hi1 + BM - 1) / BM, nqt) : qt_begin;
  }

  for (int h = hk * a.G; h < (hk + 1) * a.G; ++h) {
    const T* Q = static_cast<const T*>(args.q) + b * args.sq.b + h * args.sq.h;
    const T* dO = static_cast<const T*>(args.dout) + b * args.sdo.b + h * args.sdo.h;
    const float* LSE = args.lse + b * args.lse_sb + h * args.lse_sh;
    const float* DLT = args.delta + b * args.delta_sb + h * args.delta_sh;
    float* dQacc = args.dq_acc + ((int64_t)b * a.Hq + h) * a.Sq * D;

    // ALiBi in log2 units: -slope log2(e) |key - position|
    const float al2 = a.alibi ? a.alibi[h] * kLog2e : 0.f;
    for (int qt = qt_begin; qt < qt_end; ++qt) {
      const int q0 = qt * BM;
      __syncthreads();  // the previous tile's LDS readers are done
      for (int c = tid; c < BM * D / 8; c += NT) {
        const int ql = c / (D / 8), d0 = (c % (D / 8)) * 8;
        Frag<T> qv, dv8;
        if (q0 + ql < a.Sq) {
          load8(qv, Q + (int64_t)(q0 + ql) * args.sq.s + d0);
          load8(dv8, dO + (int64_t)(q0 + ql) * args.sdo.s + d0);
        } else {
          zero(qv);
          zero(dv8);
        }
        store8(q_lds + ql * RS + d0, qv);
        store8(do_lds + ql * RS + d0, dv8);
        for (int i = 0; i < 8; ++i) {
          qt_lds[(d0 + i) * TS + ql] = elem_t(qv, i);
          dot_lds[(d0 + i) * TS + ql] = elem_t(dv8, i);
        }
      }
      for (int i = tid; i < BM; i += NT) {
        const bool ok = q0 + i < a.Sq;
        lse_lds[i] = ok ? LSE[q0 + i] * kLog2e : 0.f;
        dlt_lds[i] = ok ? DLT[q0 + i] : 0.f;
      }
      __syncthreads();

      for (int qb = 0; qb < QB; ++qb) {
        f32x16 sacc = zeros16(), dpacc = zeros16();
        for (int s = 0; s < DS; ++s) {
          Frag<T> qa, da;
          load8(qa, q_lds + (32 * qb + r32) * RS + 16 * s + 8 * g);
          load8(da, do_lds + (32 * qb + r32) * RS + 16 * s + 8 * g);
          mma(sacc, qa, kf[s]);
          mma(dpacc, da, vf[s]);
        }
        // lane (key, half g), register r -> query row 32 qb + 8 (r/4) + 4 g + r%4
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
          const int qi = q0 + ql;
          const bool vis = qi >= rlo && qi < rhi;
          float x = sacc[r] * cs, dcap = 1.f;
          if (capped) {
            const float t = tanhf(sacc[r] * cap_in);
            x = t * cap_out;
            dcap = 1.f - t * t;
          }
          if (MASK && vis) x += a.mask[b * a.mask_sb + h * a.mask_sh + (int64_t)qi * a.mask_sq + key] * kLog2e;
          if (a.alibi) x -= al2 * fabsf((float)((int64_t)key - a.q_offset - qi));
          const float p = vis ? fast_exp2(x - lse_lds[ql]) : 0.f;
          const float dm = p * (dpacc[r] - dlt_lds[ql]);  // the gradient of the additive term
          sacc[r] = p;
          dpacc[r] = dm * dcap;
          if (MASK && args.dbias && vis) {  // the mask's gradient (a learnable score bias), added in
            float* db = args.dbias + b * args.dbias_sb + h * args.dbias_sh + (int64_t)qi * args.dbias_sq + key;
            if (args.dbias_atomic)
              __hip_atomic_fetch_add(db, dm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
              *db += dm;
          }
        }
        // dV += P^T dO and dK += dS^T Q over this 32-row block, 16 rows per step:
        // registers 8 hh .. 8 hh + 7 hold rows 16 hh + {4 g .. 4 g + 3} and
        // 16 hh + 8 + {4 g .. 4 g + 3}; the B operand reads the same rows of column d.
        for (int hh = 0; hh < 2; ++hh) {
          Frag<T> pa, dsa;
          pack8(pa, sacc, 8 * hh);
          pack8(dsa, dpacc, 8 * hh);
          for (int db = 0; db < DB; ++db) {
            const int col = 32 * qb + 16 * hh + 4 * g;
            Frag<T> dob, qb8;
            const T* dr = dot_lds + (32 * db + r32) * TS + col;
            const T* qr = qt_lds + (32 * db + r32) * TS + col;
            load4x2(dob, dr, dr + 8);
            load4x2(qb8, qr, qr + 8);
            mma(dv[db], pa, dob);
            mma(dk[db], dsa, qb8);
          }
        }
        // stage dS (as the operand dtype) for the dQ product: ds_lds[row][key]
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
          ds_lds[ql * SS + 32 * wave + r32] = from_f32<T>(dpacc[r]);
        }
      }
      __syncthreads();

      // dQ[rows, d] += dS[rows, keys] K[keys, d] over the tile's BN keys; the
      // QB x DB output blocks are shared out over the waves.
      for (int t = wave; t < QB * DB; t += NW) {
        const int qb = t / DB, db = t % DB;
        f32x16 acc = zeros16();
        for (int s = 0; s < BN / 16; ++s) {
          Frag<T> da, kb8;
          load8(da, ds_lds + (32 * qb + r32) * SS + 16 * s + 8 * g);
          load8(kb8, kt_lds + (32 * db + r32) * KTS + 16 * s + 8 * g);
          mma(acc, da, kb8);
        }
        // lane (d = 32 db + r32, half g), register r -> row 32 qb + 8 (r/4) + 4 g + r%4
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
          if (qi < a.Sq) atomic_add_f32(dQacc + (int64_t)qi * D + 32 * db + r32, acc[r]);
        }
      }
    }
  }

  // dK (scaled) and dV for this wave's keys: accumulator row = key, column = d
  for (int db = 0; db < DB; ++db) {
    for (int r = 0; r < 16; ++r) {
      const int kk = n0 + 32 * wave + 8 * (r >> 2) + 4 * g + (r & 3);
      if (kk >= a.Sk) continue;
      const int d = 32 * db + r32;
      const float vk = dk[db][r] * a.scale, vv = dv[db][r];
      if (args.accumulate) {
        float* pk = static_cast<float*>(args.dk) + b * args.sdk.b + hk * args.sdk.h + (int64_t)kk * args.sdk.s + d;
        float* pv = static_cast<float*>(args.dv) + b * args.sdv.b + hk * args.sdv.h + (int64_t)kk * args.sdv.s + d;
        *pk += vk;
        *pv += vv;
      } else {
        T* pk = static_cast<T*>(args.dk) + b * args.sdk.b + hk * args.sdk.h + (int64_t)kk * args.sdk.s + d;
        T* pv = static_cast<T*>(args.dv) + b * args.sdv.b + hk * args.sdv.h + (int64_t)kk * args.sdv.s + d;
        *pk = from_f32<T>(vk);
        *pv = from_f32<T>(vv);
      }
    }
  }
}

template <typename T, int D, int NW>
hipError_t launch_bwd_t(const BwdArgs& args, hipStream_t stream) {
  const dim3 grid((args.a.Sk + 32 * NW - 1) / (32 * NW), args.a.Hkv, args.a.B);
  const dim3 block(NW * 64);
  if (args.a.mask != nullptr)
    hipLaunchKernelGGL((bwd_kernel<T, D, NW, true>), grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL((bwd_kernel<T, D, NW, false>), grid, block, 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& args, int is_bf16, hipStream_t stream) {
  if (is_bf16)
    return args.a.D == 64 ? launch_bwd_t<bf16, 64, 4>(args, stream) : launch_bwd_t<bf16, 128, 4>(args, stream);
  return args.a.D == 64 ? launch_bwd_t<float, 64, 4>(args, stream) : launch_bwd_t<float, 128, 4>(args, stream);
}

}  // namespace fa
