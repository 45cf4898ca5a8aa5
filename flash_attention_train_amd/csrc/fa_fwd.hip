// fa_fwd.hip -- forward of the fused attention op: O and the per-row LSE.
//
// Tiled online-softmax attention (the forward half of the flash-attention
// training op on the "Flash Attn Training" skill page, section 6, trap 3: the
// forward emits O together with the LSE the backward recomputes P from).
//
// Work split: one workgroup of 4 waves per (batch, query head, 128-row query
// tile); each wave owns 32 query rows and walks the key tiles (64 keys each) that
// can be visible to its tile. K and V^T tiles are staged in LDS and shared by the
// four waves; Q stays in registers for the whole walk.
//
// Layout trick: the wave computes S^T = K Q^T (keys as rows), so in the
// accumulator every lane holds ONE query row and 16 keys of it. The row max/sum
// then need a single cross-lane step (lane l with lane l ^ 32), the probabilities
// feed the next product straight from registers as its B operand, and the
// output is accumulated transposed, O^T = V^T P^T, so the per-row rescale is a
// per-lane scalar.
//
// Numerics: scores are scaled by scale * log2(e) and exponentiated with the
// hardware exp2 (with a logit softcap c, the scaled product x first becomes
// c tanh(x / c), before the mask and ALiBi are added); the LSE is converted back to natural
// log on output. The keys a row sees by the structure (sequence end, key and query lengths,
// causal diagonal, window) come from the same range helper the bf16 kernels use. A row that
// has seen no visible key keeps m = -inf; its exponent base is taken as 0 so that
// exp2(-inf) = 0 flows through without NaN, and the epilogue writes O = 0 and
// LSE = 0 for it (skill page, section 6, trap 9). An attention sink (one more logit per head
// with no value row, llama.cpp pull request 57's list of score modifiers) joins the row sum
// in the epilogue; a row that saw no key then has O = 0 and LSE = the sink.
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

template <typename T, int D, bool MASK>
__global__ __launch_bounds__(256, 1) void fwd_kernel(const FwdArgs args) {
  constexpr int BM = 128;              // query rows per workgroup (32 per wave)
  constexpr int BN = 64;               // keys per tile
  constexpr int PAD = 16 / sizeof(T);  // 16 bytes of row padding against bank conflicts
  constexpr int KS = D + PAD;          // row stride of the K tile [BN][D]
  constexpr int VS = BN + PAD;         // row stride of the V^T tile [D][BN]
  constexpr int DS = D / 16;           // k-slot groups along the head dim
  constexpr int DB = D / 32;           // 32-wide output blocks along the head dim
  __shared__ __attribute__((aligned(16))) T k_lds[BN * KS];
  __shared__ __attribute__((aligned(16))) T vt_lds[D * VS];

  const AttnShape& a = args.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int b = blockIdx.z, h = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;  // the longest causal tiles start first
  const int q0 = qt * BM;
  const int qrow = q0 + wave * 32 + r32;
  const int hk = h / a.G;
  const float cs = a.scale * kLog2e;
  const bool capped = a.softcap > 0.f;
  const float cap_in = capped ? a.scale / a.softcap : 0.f, cap_out = a.softcap * kLog2e;

  const T* Q = static_cast<const T*>(args.q) + b * args.sq.b + h * args.sq.h;
  const T* K = static_cast<const T*>(args.k) + b * args.sk.b + hk * args.sk.h;
  const T* V = static_cast<const T*>(args.v) + b * args.sv.b + hk * args.sv.h;
  const float* Mrow = nullptr;
  if (MASK && qrow < a.Sq) Mrow = a.mask + b * a.mask_sb + h * a.mask_sh + (int64_t)qrow * a.mask_sq;
  // ALiBi in log2 units: -slope log2(e) |key - position|
  const float al2 = a.alibi ? a.alibi[h] * kLog2e : 0.f;
  const int64_t pos = a.q_offset + qrow;
  // the keys this lane's row sees by the structure, and the tiles the workgroup's rows see
  const int klen = klen_of(a, b), qlen = qlen_of(a, b);
  int64_t lo, hi;
  key_range(a, klen, qlen, qrow, lo, hi);

  // Q as the B operand of S^T = K Q^T: lane (row r32, half g) holds d = 16 s + 8 g + j
  Frag<T> qf[DS];
  for (int s = 0; s < DS; ++s) {
    if (qrow < a.Sq)
      load8(qf[s], Q + (int64_t)qrow * args.sq.s + 16 * s + 8 * g);
    else
      zero(qf[s]);
  }

  f32x16 oacc[DB];
  for (int db = 0; db < DB; ++db) oacc[db] = zeros16();
  float m = neg_inf();  // running row max (log2 units), identical in lanes l and l ^ 32
  float l = 0.f;        // this lane's share of the running row sum

  const int nkt = (a.Sk + BN - 1) / BN;
  int kt_begin = 0, kt_end = 0;
  if (q0 < qlen) {  // from the first row's lower end to the last visible row's upper end
    int64_t lo0, hi0, lo1, hi1;
    key_range(a, klen, qlen, q0, lo0, hi0);
    key_range(a, klen, qlen, min(q0 + BM, qlen) - 1, lo1, hi1);
    kt_begin = (int)min<int64_t>(lo0 / BN, nkt);
    kt_end = hi1 > lo0 ? (int)min<int64_t>((hi1 + BN - 1) / BN, nkt) : kt_begin;
  }

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    __syncthreads();  // every wave is done with the previous tile
    for (int c = tid; c < BN * D / 8; c += 256) {
      const int key = c / (D / 8), d0 = (c % (D / 8)) * 8;
      const int kg = kt * BN + key;
      Frag<T> kv, vv;
      if (kg < a.Sk) {
        load8(kv, K + (int64_t)kg * args.sk.s + d0);
        load8(vv, V + (int64_t)kg * args.sv.s + d0);
      } else {
        zero(kv);
        zero(vv);
      }
      store8(k_lds + key * KS + d0, kv);
      for (int i = 0; i < 8; ++i) vt_lds[(d0 + i) * VS + key] = elem_t(vv, i);
    }
    __syncthreads();

    // S^T for two 32-key blocks: lane (query r32, half g), register r -> key 8 (r/4) + 4 g + r%4
    f32x16 st[2];
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = zeros16();
      for (int s = 0; s < DS; ++s) {
        Frag<T> kf;
        load8(kf, k_lds + (32 * kb + r32) * KS + 16 * s + 8 * g);
        mma(st[kb], kf, qf[s]);
      }
    }

    float mx = neg_inf();
    for (int kb = 0; kb < 2; ++kb) {
      for (int r = 0; r < 16; ++r) {
        const int key = kt * BN + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
        float x = capped ? tanhf(st[kb][r] * cap_in) * cap_out : st[kb][r] * cs;
        const bool vis = key >= lo && key < hi;
        if (MASK && vis && Mrow) x += Mrow[key] * kLog2e;
        if (a.alibi) x -= al2 * fabsf((float)(key - pos));
        x = vis ? x : neg_inf();
        st[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx);
    const float base = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = fast_exp2(m - base);  // 0 while nothing was visible yet
    m = m_new;

    float ls = 0.f;
    for (int kb = 0; kb < 2; ++kb) {
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(st[kb][r] - base);
        st[kb][r] = p;
        ls += p;
      }
    }
    l = l * alpha + ls;
    for (int db = 0; db < DB; ++db)
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    // O^T += V^T P^T. Registers 8 hh .. 8 hh + 7 of key block kb hold keys
    // 32 kb + 16 hh + {4 g .. 4 g + 3} and 32 kb + 16 hh + 8 + {4 g .. 4 g + 3};
    // the V^T operand reads the same keys for its output row d.
    for (int kb = 0; kb < 2; ++kb) {
      for (int hh = 0; hh < 2; ++hh) {
        Frag<T> pf;
        pack8(pf, st[kb], 8 * hh);
        for (int db = 0; db < DB; ++db) {
          const T* row = vt_lds + (32 * db + r32) * VS + 32 * kb + 16 * hh + 4 * g;
          Frag<T> vf;
          load4x2(vf, row, row + 8);
          mma(oacc[db], vf, pf);
        }
      }
    }
  }

  // epilogue: O = acc / l, LSE = ln(sum) + max; fully masked rows -> 0 and 0 (the sink, when
  // there is one, joins the sum at the larger of its logit and the row max)
  float lt = halves_sum(l), inv, lse;
  const float sb = args.sinks ? args.sinks[h] * kLog2e : neg_inf();
  if (sb != neg_inf()) {
    const float nb = fmaxf(m, sb);
    const float fo = m == neg_inf() ? 0.f : fast_exp2(m - nb);
    lt = lt * fo + fast_exp2(sb - nb);
    inv = fo / lt;
    lse = m == neg_inf() ? args.sinks[h] : (nb + log2f(lt)) * kLn2;
  } else {
    const bool full = (m == neg_inf());
    inv = full ? 0.f : 1.f / lt;
    lse = full ? 0.f : (m + log2f(lt)) * kLn2;
  }
  if (qrow < a.Sq) {
    T* O = static_cast<T*>(args.o) + b * args.so.b + h * args.so.h + (int64_t)qrow * args.so.s;
    for (int db = 0; db < DB; ++db)
      for (int r = 0; r < 16; ++r) O[32 * db + 8 * (r >> 2) + 4 * g + (r & 3)] = from_f32<T>(oacc[db][r] * inv);
    if (g == 0) args.lse[b * args.lse_sb + h * args.lse_sh + qrow] = lse;
  }
}

template <typename T, int D>
hipError_t launch_fwd_t(const FwdArgs& args, hipStream_t stream) {
  const dim3 grid((args.a.Sq + 127) / 128, args.a.Hq, args.a.B);
  const dim3 block(256);
  if (args.a.mask != nullptr)
    hipLaunchKernelGGL((fwd_kernel<T, D, true>), grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, false>), grid, block, 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& args, int is_bf16, hipStream_t stream) {
  if (is_bf16) return args.a.D == 64 ? launch_fwd_t<bf16, 64>(args, stream) : launch_fwd_t<bf16, 128>(args, stream);
  return args.a.D == 64 ? launch_fwd_t<float, 64>(args, stream) : launch_fwd_t<float, 128>(args, stream);
}

}  // namespace fa
