// fa_kernels.h -- kernel argument blocks and launcher declarations (internal).
//
// The C ABI layer validates every argument on the host, fills one of these
// blocks and calls the matching launcher; the launchers pick a template instance
// and enqueue it on the caller's stream. Strides are in elements of each tensor's
// own type.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct Strides {
  int64_t b, h, s;
};

struct AttnShape {
  int B, Hq, Hkv, Sq, Sk, D;
  int G;             // Hq / Hkv
  int causal;
  int64_t q_offset;  // key position of query row 0
  float scale;       // multiplies <q, k>
  const float* mask; // additive [b][h][i][j] fp32 or nullptr (b and h strides 0: shared)
  int64_t mask_sb, mask_sq;
  int64_t mask_sh;   // head stride of the mask: 0 = one mask for every head, else a score bias per head
  const uint8_t* tiles;      // mask block classes [Bm][ceil(Sq/64)][ceil(Sk/64)] or nullptr
  const uint64_t* rowbits;   // per block, 64 words: bit j of word i = entry (i, j) visible
  const uint64_t* colbits;   // per block, 64 words: bit i of word j = entry (i, j) visible
  int tiles_bstride;         // blocks per mask batch entry (0 when the mask is shared)
  int tiles_ncol;            // ceil(Sk / 64)
  // structured masks: entry (b, i, j) is hidden when j >= klen(b), i >= qlen(b),
  // j < q_offset + i - wl (wl >= 0) or j > q_offset + i + wr (wr >= 0)
  const int32_t* key_len;    // [B] or nullptr (Sk)
  const int32_t* q_len;      // [B] or nullptr (Sq)
  int wl, wr;                // window bounds, -1: none
  // ALiBi: score (h, i, j) gets -alibi[h] |j - (q_offset + i)|; or nullptr. It runs in the
  // masked kernels' bias body (every live block counts as a bias block)
  const float* alibi;
  // logit softcap c (> 0) or 0: the scaled product x becomes c tanh(x / c) before the mask
  // and ALiBi are added
  float softcap;
  // storage of K and V for the bf16 kernels: kKvBf16 (the compute dtype), kKvF16 (fp16), or
  // kKvQ8 (q8_0: int8 quants, one fp16 scale per 32 values along D at kscale / vscale,
  // element strides sks / svs); the walks convert each tile to bf16 as they read it
  int kvf;
  const _Float16* kscale;
  const _Float16* vscale;
  Strides sks, svs;
};
constexpr int kKvBf16 = 0, kKvF16 = 1, kKvQ8 = 2;

// the structured lengths of batch entry b (clamped to the tensor lengths)
__device__ __forceinline__ int klen_of(const AttnShape& a, int b) {
  return a.key_len ? min(max(a.key_len[b], 0), a.Sk) : a.Sk;
}
__device__ __forceinline__ int qlen_of(const AttnShape& a, int b) {
  return a.q_len ? min(max(a.q_len[b], 0), a.Sq) : a.Sq;
}
// keys [lo, hi) that query row i can see by the structure alone (sequence ends, key length,
// causal diagonal, window); empty when the row is past the query length
__host__ __device__ __forceinline__ void key_range(const AttnShape& a, int klen, int qlen, int64_t i, int64_t& lo,
                                          int64_t& hi) {
  const int64_t pos = a.q_offset + i;
  lo = a.wl >= 0 ? pos - a.wl : 0;
  hi = klen;
  if (a.causal && pos + 1 < hi) hi = pos + 1;
  if (a.wr >= 0 && pos + a.wr + 1 < hi) hi = pos + a.wr + 1;
  if (lo < 0) lo = 0;
  if (i >= qlen || hi < lo) hi = lo;
}
// rows [lo, hi) that can see key j by the structure alone
__host__ __device__ __forceinline__ void row_range(const AttnShape& a, int klen, int qlen, int64_t j, int64_t& lo,
                                          int64_t& hi) {
  lo = 0;
  hi = qlen;
  if (a.causal && j - a.q_offset > lo) lo = j - a.q_offset;            // j <= q_offset + i
  if (a.wr >= 0 && j - a.q_offset - a.wr > lo) lo = j - a.q_offset - a.wr;
  if (a.wl >= 0 && j - a.q_offset + a.wl + 1 < hi) hi = j - a.q_offset + a.wl + 1;  // j >= q_offset + i - wl
  if (j >= klen || hi < lo) hi = lo;
}

// block classes: dead = all -inf, open = all 0, bits = only 0 / -inf, bias = finite biases
constexpr int kTileDead = 0, kTileOpen = 1, kTileBits = 2, kTileBias = 3, kMaskTile = 64;

__device__ __forceinline__ int tile_index(const AttnShape& a, int b, int rt, int ct) {
  return b * a.tiles_bstride + rt * a.tiles_ncol + ct;
}
// class of mask block (b, row block rt, key block ct); "bias" (read every value) without a
// map. Read through the constant address space, one aligned dword (the class array is
// 256-byte aligned and padded to a multiple of 256 bytes): a wave-uniform index becomes a
// scalar load, tracked apart from the vector memory counter that orders the
// direct-to-LDS tile loads; a per-lane index becomes a vector load.
__device__ __forceinline__ int tile_class(const AttnShape& a, int b, int rt, int ct) {
  if (!a.tiles) return kTileBias;
  const int i = tile_index(a, b, rt, ct);
  const auto* w = reinterpret_cast<const __attribute__((address_space(4))) uint32_t*>(
      reinterpret_cast<uintptr_t>(a.tiles) + (uintptr_t)(i & ~3));
  return (int)((*w >> (8 * (i & 3))) & 0xffu);
}

// The classes of 64 consecutive mask blocks along a walk (the row blocks of one key
// column for a dK/dV wave, the key blocks of one row block for a forward or dQ wave), one
// per lane, fetched by one vector load per 64 blocks. A step reads its block's class with
// one readlane and loads its visibility word only when the block is 0 / -inf, instead of
// issuing both loads (and their 64-bit address arithmetic) for every step.
struct ClassRun {
  int cls;   // class of block base + lane
  int base;  // walk position of lane 0's block (a multiple of 64), or -64 before the first load
  // lane l takes the class of block index(base + l), or dead when base + l >= n
  template <class Index>
  __device__ __forceinline__ void load(const AttnShape& a, int new_base, int n, Index&& index) {
    const auto* t =
        reinterpret_cast<const __attribute__((address_space(1))) uint8_t*>(reinterpret_cast<uintptr_t>(a.tiles));
    const int pos = new_base + (int)(threadIdx.x & 63);
    cls = pos < n ? (int)t[index(pos)] : kTileDead;
    base = new_base;
  }
  // class of the block at walk position pos (base <= pos < base + 64), wave-uniform
  __device__ __forceinline__ int at(int pos) const { return __builtin_amdgcn_readlane(cls, pos - base); }
};


// The live candidates of a walk (candidate j = 0 .. n - 1), 256 at a time as bit words
// in LDS: every thread tests one candidate, so that no step of the walk waits on a class
// load. The walk is workgroup-uniform, and every call is made by the whole workgroup at
// the same point.
struct LiveWords {
  static constexpr int kThreads = 256, kWaves = 4;  // the workgroup: four waves
  uint64_t* words;  // [kWaves] in LDS
  int base;
  uint64_t w[kWaves];  // the words of candidates base .. base + kThreads - 1, kept wave-uniform
  template <class F>
  __device__ __forceinline__ int next(int j, int n, int tid, F&& live) {
    while (j < n) {
      if (j >= base + kThreads) {
        const int c = (j & ~(kThreads - 1)) + tid;
        const uint64_t bw = __ballot(c < n && live(c));
        __syncthreads();  // the previous words are no longer read
        if ((tid & 63) == 0) words[tid >> 6] = bw;
        __syncthreads();
        base = j & ~(kThreads - 1);
        // read once into scalar registers, so that a step of the walk finds its next
        // candidate without an LDS read (whose wait would also wait for every LDS read
        // issued before it)
        #pragma unroll
        for (int k = 0; k < kWaves; ++k) {
          const uint64_t x = words[k];
          w[k] = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32) |
                 __builtin_amdgcn_readfirstlane((uint32_t)x);
        }
      }
      const int off = j - base, k = off >> 6;
      const uint64_t wk = k == 0 ? w[0] : k == 1 ? w[1] : k == 2 ? w[2] : w[3];
      const uint64_t bits = wk >> (off & 63);
      if (bits) return j + (int)__builtin_ctzll(bits);
      j = base + 64 * (k + 1);
    }
    return n;
  }
};

// bf16 backward decomposition: waves per workgroup (one wave per SIMD: 1024 / kBwdWaves
// workgroups fill the GPU), keys per dK/dV workgroup and query rows per dQ workgroup
constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdUnit = 32 * kBwdWaves;
// keys per dK/dV workgroup of the role-split walk (two 32-key groups, two roles each)
constexpr int kBwdRoleKeys = 64;
// bytes of one stored dS block: a 64-row query tile times a dK/dV workgroup's keys, bf16
constexpr int kDsBlock = 64 * kBwdUnit * 2;
// query rows per workgroup of the dQ pass over stored dS (one 64-row tile per wave)
constexpr int kDsRows = 64 * kBwdWaves;

struct FwdArgs {
  AttnShape a;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  Strides sq, sk, sv, so;
  int64_t lse_sb, lse_sh;
  float inv_scale;  // 1 / scale (scale > 0)
  int mask_vec4;    // the mask can be read 4 floats at a time (16-byte aligned rows)
  const float* sinks;  // [Hq] sink logits (natural log) joining each row's denominator, or null
  // split key walks (splits > 1): workgroup z walks the z-th share of the key tiles and
  // stores its O rows normalised by its own row sum (bf16) and (base, row sum) per row,
  // merged afterwards
  int splits;
  void* part_o;     // bf16 [splits][B][Hq][Sq][D]: the share's rows normalised by its own row sum
  float* part_ml;   // [splits][B][Hq][Sq][2]: exponent base (log2 units, -inf: no key), row sum
};

struct PreArgs {
  int B, Hq, Sq, D;
  const void* o;
  const void* dout;
  float* delta;
  Strides so, sdo;
  int64_t delta_sb, delta_sh;
};

// dsink[h] += -sum over the head's rows of exp(sinks[h] - LSE) * Delta
struct SinkArgs {
  int B, Hq, Sq;
  const float* sinks;
  const float* lse;
  const float* delta;
  int64_t lse_sb, lse_sh, delta_sb, delta_sh;
  float* dsink;
};

struct BwdArgs {
  AttnShape a;
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* delta;
  void* dk;        // dtype output (plain) or fp32 accumulator (chunked)
  void* dv;
  float* dq_acc;   // fp32 [B, Hq, Sq, D] contiguous workspace, zeroed before the launch
  Strides sq, sk, sv, sdo, sdk, sdv;
  int64_t lse_sb, lse_sh, delta_sb, delta_sh;
  int accumulate;  // 1: dK/dV are fp32 accumulators and receive +=, 0: overwrite in dtype
  float inv_scale; // 1 / scale
  int mask_vec4;   // the mask can be read 4 floats at a time
  // the mask's gradient (fp32, added into, broadcast like the mask) or null; dbias_atomic:
  // several heads or batch entries add into one entry; dbias_vec4: 16-byte rows of 4 entries
  float* dbias;
  int64_t dbias_sb, dbias_sh, dbias_sq;
  int dbias_atomic, dbias_vec4;
};

// unit -> (key tile, batch, kv head, split) of a dK/dV workgroup; key tiles vary slowest so
// that the long causal tiles (small key index) are dispatched first
struct KvUnit {
  int kt, b, hk, split;
};
// unit -> (query tile, batch, head, split, splits) of a dQ workgroup; the last query tiles
// (longest under a causal mask) are dispatched first, the whole tiles before the
// q_tiles_split first ones, which are each walked by q_split workgroups and dispatched last
struct QUnit {
  int qt, b, h, split, nsplit;
};

// Work decomposition of the bf16 backward (one launch, two kinds of workgroups).
struct BwdPlan {
  int kv_split;    // workgroups sharing one key tile's dK/dV walk (> 1: fp32 partial slices)
  int q_split;     // workgroups sharing one split query tile's dQ walk (> 1: fp32 partial slices)
  int q_bm;           // query rows per dQ workgroup (kBwdUnit, or kDsRows over stored dS)
  int q_tiles_split;  // how many q_bm-row query tiles (the first ones, dispatched last) are split
                      // q_split ways; the others walk whole and store dQ directly
  int n_kv_units;  // dK/dV workgroups (launched first)
  int n_q_units;   // dQ workgroups
  int dq_separate; // 1: the dQ workgroups run as a second kernel (two per compute unit)
  int kv_role;     // 1: the role-split dK/dV walk (64-key workgroups, two per compute unit)
  float* dk_part;  // fp32 [kv_split][B, Hkv, Sk, D] partial sums when kv_split > 1
  float* dv_part;
  float* dq_part;  // fp32 [q_split][B, Hq, Sq, D] partial sums when q_split > 1
  void* dq;        // dQ output (dtype) written directly when q_split == 1
  Strides sdq;
  // dQ from stored dS (or null: the dQ walk recomputes S and dP): the dK/dV walk stores
  // every pair's dS, block (b, h, 64-row tile rt, key tile kt) of kDsBlock bytes at
  // ((b Hq + h) ds_nku + kt) ds_nrt + rt (a key tile's row tiles adjacent: the walk that
  // writes them and the four waves of a dQ workgroup that read them both stay within one
  // key tile's run), and the dQ workgroups multiply it by K
  char* ds;
  int ds_nrt, ds_nku;
  // (host side) the stream of the separate dQ kernel, or null for the launch stream
  hipStream_t dq_stream;
};

// out = scale * sum of nparts fp32 slices [B, H, S_parts, D] (slice s at parts + s * part_stride),
// over rows 0 .. S - 1 of every (b, h), stored in the output dtype, or added to an fp32 output
// when accumulate is set
struct ReduceArgs {
  int B, H, S, D;
  int S_parts;
  const float* parts;
  int nparts;
  int64_t part_stride;
  void* out;
  Strides so;
  float scale;
  int accumulate;
};

struct DqArgs {
  int B, Hq, Sq, D;
  const float* dq_acc;
  void* dq;
  Strides sdq;
  float scale;
};

// launchers: return hipSuccess or the launch error
hipError_t launch_fwd(const FwdArgs& args, int is_bf16, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs& args, int qb, hipStream_t stream);
// the split forward (args.splits > 1) followed by the merge of its partial rows
hipError_t launch_fwd_bf16_split(const FwdArgs& args, hipStream_t stream);
hipError_t launch_preprocess(const PreArgs& args, int is_bf16, hipStream_t stream);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream);
hipError_t launch_mask_tiles(const AttnShape& a, uint8_t* tiles, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& args, int is_bf16, hipStream_t stream);
hipError_t launch_dq_convert(const DqArgs& args, int is_bf16, hipStream_t stream);
// reduces args, and args1 too when given (same shape and dtype: one launch for dK and dV)
// reduces args, and args1 / args2 too when given (same D and output dtype; one launch)
hipError_t launch_reduce_parts(const ReduceArgs& args, const ReduceArgs* args1, const ReduceArgs* args2, int is_bf16,
                               hipStream_t stream);
hipError_t launch_sink_grad(const SinkArgs& args, hipStream_t stream);

// bf16 values of a q8_0 window: out[b][h][s][32 c + t] = bf16(d[b][h][s][c] * qs[b][h][s][32 c + t])
struct DequantArgs {
  int B, H, S, D;
  const int8_t* qs;
  const _Float16* d;
  void* out;  // bf16
  Strides sq, sd, so;  // element strides of qs, d and out
};
hipError_t launch_dequant_q8_0(const DequantArgs& args, hipStream_t stream);
struct ConvertArgs {
  int B, H, S, D;
  const _Float16* src;
  void* out;  // fp32 or bf16
  int to_bf16;
  Strides ss, so;  // element strides of src and out
};
hipError_t launch_convert_f16(const ConvertArgs& args, hipStream_t stream);
// dq_ds: dQ from stored dS (dQ units of kDsRows rows; q_tiles_split counts kBwdUnit-row tiles
// and is rounded up to whole units)
void plan_bwd_bf16(const AttnShape& a, int kv_split, int q_split, int q_tiles_split, int dq_separate,
                   BwdPlan* plan, int kv_role, int dq_ds = 0);

__host__ __device__ __forceinline__ KvUnit kv_unit_of(const AttnShape& a, const BwdPlan& plan, int unit) {
  const int per_tile = a.B * a.Hkv * plan.kv_split;
  int rem = unit % per_tile;
  const int split = rem % plan.kv_split;
  rem /= plan.kv_split;
  return {unit / per_tile, rem / a.Hkv, rem % a.Hkv, split};
}
__host__ __device__ __forceinline__ QUnit q_unit_of(const AttnShape& a, const BwdPlan& plan, int unit) {
  const int nqt = (a.Sq + plan.q_bm - 1) / plan.q_bm;
  const int bh = a.B * a.Hq;
  const int n_whole = (nqt - plan.q_tiles_split) * bh;
  if (unit < n_whole) {
    const int rem = unit % bh;
    return {nqt - 1 - unit / bh, rem / a.Hq, rem % a.Hq, 0, 1};
  }
  unit -= n_whole;
  const int per_tile = bh * plan.q_split;
  int rem = unit % per_tile;
  const int split = rem % plan.q_split;
  rem /= plan.q_split;
  return {plan.q_tiles_split - 1 - unit / per_tile, rem / a.Hq, rem % a.Hq, split, plan.q_split};
}
hipError_t launch_bwd_bf16(const BwdArgs& args, const BwdPlan& plan, hipStream_t stream);

}  // namespace fa
