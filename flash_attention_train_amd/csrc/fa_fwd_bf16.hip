// fa_fwd_bf16.hip -- the bf16 forward: O and the per-row LSE.
//
// Same mathematics as the generic forward (online softmax over key tiles, the
// LSE kept for the backward -- "Flash Attn Training" skill page, section 6,
// trap 3), organised for gfx950's matrix cores and LDS:
//
//  * one workgroup of 4 waves per (batch, head, 32*4*QB-row query tile); each
//    wave owns QB blocks of 32 query rows, held in registers as the B operand
//    of S^T = K Q^T for the whole walk;
//  * K and V tiles of BN keys are staged row-major in LDS, double-buffered: the
//    next tile's global loads are issued before the current tile's products and
//    written to the other buffer afterwards, so one barrier per tile suffices;
//  * K fragments are 16-byte row reads; the V^T operand of O^T = V^T P^T comes
//    from the row-major V tile through the LDS transpose read
//    (ds_read_b64_tr_b16: in each 16-lane group, lane L addresses row
//    r0 + L/4, column c0 + 4 (L % 4) and lane i receives column c0 + i of rows
//    r0 .. r0 + 3), so V never needs a transposed copy;
//  * each K or V fragment read from LDS feeds QB matrix products;
//  * the running max is updated lazily: the exponent base only moves (and O and
//    the row sum are only rescaled) when a row's max grows by more than 8 in
//    log2 units, so probabilities stay below 2^8 and most tiles skip the
//    rescale; the final O = acc / l and LSE = base + log2(l) are exact either way;
//  * element masks (sequence tail, causal diagonal) are applied only on tiles
//    that need them; the additive mask, when given, is read 4 keys at a time.
// A row that sees no key keeps base = -inf and ends with O = 0, LSE = 0 (skill
// page, section 6, trap 9).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ f32x16 zeros16() {
  f32x16 z;
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// One transposed 4 x 16 read: lane i of each 16-lane group gets column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 tr_read(const bf16* lds_base, int elem_offset) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) bf16*)lds_base + elem_offset));
}

template <int D, int QB, int BN, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1) void fwd_bf16_kernel(const FwdArgs args) {
  constexpr int NW = 4;
  constexpr int BM = NW * QB * 32;  // query rows per workgroup
  constexpr int KB = BN / 32;       // 32-key blocks per tile
  constexpr int KS = D + 8;         // LDS row stride (elements): 16 bytes of padding
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int CH = BN * D / 8;    // 16-byte chunks per tile
  constexpr int CPT = CH / 256;     // chunks per thread
  __shared__ __attribute__((aligned(16))) bf16 k_lds[2][BN * KS];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[2][BN * KS];

  const AttnShape& a = args.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int b = blockIdx.z, h = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;  // longest causal tiles first
  const int q0 = qt * BM;
  const int qw = q0 + wave * QB * 32;          // first row of this wave
  const int hk = h / a.G;
  const float cs = a.scale * kLog2e;           // scale > 0 (checked on the host)

  const bf16* Q = static_cast<const bf16*>(args.q) + b * args.sq.b + h * args.sq.h;
  const bf16* K = static_cast<const bf16*>(args.k) + b * args.sk.b + hk * args.sk.h;
  const bf16* V = static_cast<const bf16*>(args.v) + b * args.sv.b + hk * args.sv.h;

  // Q rows as B operands: lane (row r32, half g) holds d = 16 s + 8 g .. + 7
  bf16x8 qf[QB][DS];
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw + 32 * qb + r32;
    for (int s = 0; s < DS; ++s) {
      if (row < a.Sq)
        qf[qb][s] = *reinterpret_cast<const bf16x8*>(Q + (int64_t)row * args.sq.s + 16 * s + 8 * g);
      else
        zero(qf[qb][s]);
    }
  }

  f32x16 oacc[QB][DB];
  float base[QB], lsum[QB];
  for (int qb = 0; qb < QB; ++qb) {
    for (int db = 0; db < DB; ++db) oacc[qb][db] = zeros16();
    base[qb] = neg_inf();
    lsum[qb] = 0.f;
  }

  const int nkt = (a.Sk + BN - 1) / BN;
  int kt_end = nkt;
  if (CAUSAL) {
    const int64_t last_key = a.q_offset + q0 + BM - 1;
    kt_end = last_key < 0 ? 0 : (int)((last_key / BN + 1) < nkt ? (last_key / BN + 1) : nkt);
  }

  // tile loader: thread tid moves chunks tid + 256 i (row = chunk / (D/8))
  bf16x8 kpre[CPT], vpre[CPT];
  auto load_tile = [&](int kt) {
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const int key = kt * BN + c / (D / 8), d0 = (c % (D / 8)) * 8;
      if (key < a.Sk) {
        kpre[i] = *reinterpret_cast<const bf16x8*>(K + (int64_t)key * args.sk.s + d0);
        vpre[i] = *reinterpret_cast<const bf16x8*>(V + (int64_t)key * args.sv.s + d0);
      } else {
        zero(kpre[i]);
        zero(vpre[i]);
      }
    }
  };
  auto store_tile = [&](int buf) {
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / 8), d0 = (c % (D / 8)) * 8;
      *reinterpret_cast<bf16x8*>(&k_lds[buf][row * KS + d0]) = kpre[i];
      *reinterpret_cast<bf16x8*>(&v_lds[buf][row * KS + d0]) = vpre[i];
    }
  };

  if (kt_end > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  // transpose-read addressing inside a 16-lane group
  const int G16 = lane >> 4, L16 = lane & 15;
  const int tr_row = L16 >> 2, tr_col = 16 * (G16 & 1) + 4 * (L16 & 3);

  for (int kt = 0; kt < kt_end; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < kt_end;
    if (more) load_tile(kt + 1);
    const bf16* kb_lds = k_lds[buf];
    const bf16* vb_lds = v_lds[buf];

    // S^T = K Q^T for both 32-key blocks; each K fragment serves all QB query blocks
    f32x16 st[QB][KB];
    for (int qb = 0; qb < QB; ++qb)
      for (int kb = 0; kb < KB; ++kb) st[qb][kb] = zeros16();
    for (int kb = 0; kb < KB; ++kb) {
      for (int s = 0; s < DS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb_lds + (32 * kb + r32) * KS + 16 * s + 8 * g);
        for (int qb = 0; qb < QB; ++qb) mma(st[qb][kb], kf, qf[qb][s]);
      }
    }

    // does this tile need per-element masking (sequence tail / causal diagonal)?
    const int key0 = kt * BN;
    bool edge = key0 + BN > a.Sk;
    if (CAUSAL) edge = edge || ((int64_t)key0 + BN - 1 > a.q_offset + qw);

    bf16x8 pf[QB][KB][2];
    for (int qb = 0; qb < QB; ++qb) {
      const int row = qw + 32 * qb + r32;
      if (MASK || edge) {
        const float* Mrow = nullptr;
        if (MASK && row < a.Sq) Mrow = a.mask + b * a.mask_sb + (int64_t)row * a.mask_sq;
        for (int kb = 0; kb < KB; ++kb) {
          for (int rr = 0; rr < 4; ++rr) {
            const int k4 = key0 + 32 * kb + 8 * rr + 4 * g;  // 4 consecutive keys k4 .. k4 + 3
            float mv[4] = {0.f, 0.f, 0.f, 0.f};
            if (MASK && Mrow) {
              if (k4 + 3 < a.Sk && args.mask_vec4) {
                const f32x4 m4 = *reinterpret_cast<const f32x4*>(Mrow + k4);
                mv[0] = m4[0]; mv[1] = m4[1]; mv[2] = m4[2]; mv[3] = m4[3];
              } else {
                for (int e = 0; e < 4; ++e) mv[e] = (k4 + e < a.Sk) ? Mrow[k4 + e] : 0.f;
              }
            }
            for (int e = 0; e < 4; ++e) {
              const int key = k4 + e;
              bool vis = key < a.Sk;
              if (CAUSAL) vis = vis && ((int64_t)key <= a.q_offset + row);
              // the mask enters the raw score as M / scale so that one fma applies both later
              float x = st[qb][kb][4 * rr + e];
              if (MASK) x += mv[e] * args.inv_scale;
              st[qb][kb][4 * rr + e] = vis ? x : neg_inf();
            }
          }
        }
      }
      // row max of this tile (raw score units), shared by lanes l and l ^ 32
      float mx = neg_inf();
      for (int kb = 0; kb < KB; ++kb)
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(st[qb][kb][r], st[qb][kb][r + 1]));
      mx = fmaxf(mx, xor32(mx));
      const float mscaled = mx * cs;
      const bool need = mscaled > base[qb] + 8.f;
      if (__any(need)) {
        // lanes that keep their base use alpha = 1 (their base may still be -inf);
        // a lane moving off -inf gets alpha = 0, its accumulators being empty
        const float alpha = need ? fast_exp2(base[qb] - mscaled) : 1.f;
        const float nb = need ? mscaled : base[qb];
        base[qb] = nb;
        lsum[qb] *= alpha;
        for (int db = 0; db < DB; ++db)
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
      }
      const float nbase = (base[qb] == neg_inf()) ? 0.f : -base[qb];
      float ls = 0.f;
      for (int kb = 0; kb < KB; ++kb) {
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(st[qb][kb][r], cs, nbase));
          st[qb][kb][r] = p;
          ls += p;
        }
        pack8(pf[qb][kb][0], st[qb][kb], 0);
        pack8(pf[qb][kb][1], st[qb][kb], 8);
      }
      lsum[qb] += ls;
    }

    // O^T += V^T P^T: registers 8 hh .. 8 hh + 7 of key block kb hold keys
    // 32 kb + 16 hh + 8 t + 4 g + e (t = 0, 1; e = 0..3) -- the rows each transpose read returns
    for (int kb = 0; kb < KB; ++kb) {
      for (int hh = 0; hh < 2; ++hh) {
        const int rbase = 32 * kb + 16 * hh + 4 * g + tr_row;
        for (int db = 0; db < DB; ++db) {
          const bf16x4 lo = tr_read(vb_lds, rbase * KS + 32 * db + tr_col);
          const bf16x4 hi = tr_read(vb_lds, (rbase + 8) * KS + 32 * db + tr_col);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          for (int qb = 0; qb < QB; ++qb) mma(oacc[qb][db], vf, pf[qb][kb][hh]);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: O = acc / l, LSE = (base + log2 l) ln 2; fully masked rows -> 0, 0
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw + 32 * qb + r32;
    const float lt = lsum[qb] + xor32(lsum[qb]);
    const bool full = base[qb] == neg_inf();
    const float inv = full ? 0.f : 1.f / lt;
    const float lse = full ? 0.f : (base[qb] + log2f(lt)) * kLn2;
    if (row < a.Sq) {
      bf16* O = static_cast<bf16*>(args.o) + b * args.so.b + h * args.so.h + (int64_t)row * args.so.s;
      for (int db = 0; db < DB; ++db) {
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 o4;
          for (int e = 0; e < 4; ++e) o4[e] = (bf16)(oacc[qb][db][4 * rr + e] * inv);
          *reinterpret_cast<bf16x4*>(O + 32 * db + 8 * rr + 4 * g) = o4;
        }
      }
      if (g == 0) args.lse[b * args.lse_sb + h * args.lse_sh + row] = lse;
    }
  }
}

template <int D, int QB, int BN>
hipError_t launch_t(const FwdArgs& args, hipStream_t stream) {
  constexpr int BM = 4 * QB * 32;
  const dim3 grid((args.a.Sq + BM - 1) / BM, args.a.Hq, args.a.B);
  const bool causal = args.a.causal != 0, mask = args.a.mask != nullptr;
  if (causal && mask)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BN, true, true>), grid, dim3(256), 0, stream, args);
  else if (causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BN, true, false>), grid, dim3(256), 0, stream, args);
  else if (mask)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BN, false, true>), grid, dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BN, false, false>), grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

// variant: 1 = 32 query rows per wave, 64-key tiles; 2 = 64 rows per wave, 32-key tiles
hipError_t launch_fwd_bf16(const FwdArgs& args, int variant, hipStream_t stream) {
  if (args.a.D == 64) return variant == 2 ? launch_t<64, 2, 32>(args, stream) : launch_t<64, 1, 64>(args, stream);
  return variant == 2 ? launch_t<128, 2, 32>(args, stream) : launch_t<128, 1, 64>(args, stream);
}

}  // namespace fa
