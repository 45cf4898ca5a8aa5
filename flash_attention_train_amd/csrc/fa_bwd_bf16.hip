// fa_bwd_bf16.hip -- the bf16 backward: dQ, dK, dV in one launch.
//
// The backward rebuilds P tile by tile from the forward's per-row LSE, uses the
// preprocessed Delta = rowsum(dO o O), and adds the dK/dV contributions of every
// query head of a group into the group's one KV head (llama.cpp pull request 57,
// commit 86c140d, the tiled backward). On gfx950 it is split into two kinds of
// workgroups that run side by side in one grid, so that neither needs the other's
// results and no score tile ever travels through LDS or memory:
//
//  dK/dV workgroups (KV-stationary): 4 waves x 32 keys own a 128-key tile of one
//    KV head. They walk the (query head of the group, 64-row query tile) pairs
//    that can see the keys, with the Q and dO tiles copied straight from global
//    memory into LDS (double-buffered, XOR-swizzled rows) and shared by the waves.
//    Per 32-row block:
//      S  = Q K^T, dP = dO V^T   (A: Q / dO rows from LDS, B: K / V in registers)
//      P  = exp2(S c + M log2e - LSE log2e), dS = P (dP - Delta)
//      dV += P^T dO, dK += dS^T Q  (A: P / dS straight from the accumulators,
//                                   B: dO^T / Q^T by LDS transpose reads)
//  dQ workgroups (Q-stationary): 4 waves x 32 rows own a 128-row query tile of
//    one head and walk its visible 64-key tiles (K and V staged in LDS the same
//    way), computing S^T = K Q^T and dP^T = V dO^T so that each lane holds one
//    query row; dS^T then feeds dQ += dS K directly as the A operand, with the K
//    operand read by LDS transpose reads.
//
// When the launch balances better that way, the dK/dV walk is split over several
// workgroups per key tile and the dQ walk over several per query tile; each split
// stores its fp32 partial sums into a slice of its own (no atomics), and a reduce
// pass sums the slices into the output dtype (or adds them to the chunked walk's
// window accumulators). Unsplit work stores its results directly. Masked entries get P = 0 exactly, so fully masked rows and key
// columns end with exactly zero gradients ("Flash Attn Training" skill page,
// section 6, traps 8 and 9).
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_tile.h"

namespace fa {

namespace {

constexpr int NT = kBwdThreads;  // threads per workgroup (kBwdWaves waves of 32 keys or rows)
constexpr int KV_BN = kBwdUnit;  // keys per dK/dV workgroup
constexpr int KV_BM = 64;        // query rows per staged tile of the dK/dV walk
constexpr int Q_BM = kBwdUnit;   // query rows per dQ workgroup
constexpr int Q_BN = 64;         // keys per staged tile of the dQ walk
static_assert(2 * KV_BM <= NT, "one thread per LSE / Delta value of a staged tile");
static_assert(NT == LiveWords::kThreads, "one live-candidate bit word per wave");

__device__ __forceinline__ f32x16 zeros16() {
  f32x16 z;
  #pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}


// (the unit decoding, kv_unit_of and q_unit_of, is shared with the host checker: fa_kernels.h)

// The 64-row query tiles [qt0, qt_end) a dK/dV walk over keys [n0, n0 + KV_BN) visits by the
// structure (sequence ends, causal diagonal, key and query lengths, window): from the first
// key's lower row end to the last live key's upper end (both ends move down with the key).
// The dQ walk over stored dS asks the same question to know which dS blocks were written.
__device__ __forceinline__ void kv_row_tiles(const AttnShape& a, int klen, int qlen, int n0, int& qt0, int& qt_end) {
  qt0 = 0;
  qt_end = 0;
  if (n0 < klen) {
    int64_t lo, hi, lo1, hi1;
    row_range(a, klen, qlen, n0, lo, hi);
    row_range(a, klen, qlen, min(n0 + KV_BN, klen) - 1, lo1, hi1);
    const int nqt = (a.Sq + KV_BM - 1) / KV_BM;
    qt0 = (int)min<int64_t>(lo / KV_BM, nqt);
    qt_end = hi1 > lo ? (int)min<int64_t>((hi1 + KV_BM - 1) / KV_BM, nqt) : qt0;
    if (qt_end < qt0) qt_end = qt0;
  }
}

// Does any mask block of rows [r0, r0 + nr) x keys [c0, c0 + nc) (in 64-blocks) carry
// additive values? Units whose blocks are all dead / open / 0-or--inf run a body
// compiled without the mask-value reads, which keeps their loop free of that code.
// Called by the whole workgroup: the threads test the blocks together.
__device__ __forceinline__ bool any_bias_block(const AttnShape& a, int b, int rb0, int nrb, int cb0, int ncb) {
  if (!a.tiles || a.alibi) return true;
  const int nrt = (a.Sq + kMaskTile - 1) / kMaskTile, nct = (a.Sk + kMaskTile - 1) / kMaskTile;
  nrb = min(nrb, nrt - rb0);
  ncb = min(ncb, nct - cb0);
  int any = 0;
  for (int i = threadIdx.x; i < nrb * ncb; i += NT) {
    const int rt = rb0 + i / ncb, ct = cb0 + i % ncb;
    any |= tile_class(a, b, rt, ct) == kTileBias;
  }
  return __syncthreads_or(any) != 0;
}

// Are all mask blocks of rows [r0, r0 + nr) x keys [c0, c0 + nc) (in 64-blocks) open (every
// entry 0)? Units over open blocks only run the body compiled without a mask, which has no
// block-class and visibility-word handling. Called by the whole workgroup.
__device__ __forceinline__ bool all_open_blocks(const AttnShape& a, int b, int rb0, int nrb, int cb0, int ncb) {
  if (!a.tiles || a.alibi) return false;
  const int nrt = (a.Sq + kMaskTile - 1) / kMaskTile, nct = (a.Sk + kMaskTile - 1) / kMaskTile;
  nrb = min(nrb, nrt - rb0);
  ncb = min(ncb, nct - cb0);
  int other = 0;
  for (int i = threadIdx.x; i < nrb * ncb; i += NT) {
    const int rt = rb0 + i / ncb, ct = cb0 + i % ncb;
    other |= tile_class(a, b, rt, ct) != kTileOpen;
  }
  return __syncthreads_or(other) == 0;
}

// ---------------------------------------------------------------------------
// dK / dV workgroup
// ---------------------------------------------------------------------------
// Store a wave's 32 x D fp32 accumulator block (lane (column 32 db + r32, half g),
// register r -> row 8 (r/4) + 4 g + r%4) through LDS: staged row-major, with the 32-column
// halves of every second group of 4 rows swapped so that the two lane halves of a write
// hit different banks, then read back as 16-byte row chunks and handed to
// sink.put(row, column, 4 values). One 16-byte store per chunk replaces one 2- or 4-byte
// store per element. `stage` is this wave's 32 x D floats of LDS, idle around the call;
// the wave reads back only what it wrote itself, in order.
template <int D, class Sink>
__device__ __forceinline__ void store_block(const f32x16 (&acc)[D / 32], float mul, float* stage, int lane,
                                            const Sink& sink) {
  const int g = lane >> 5, r32 = lane & 31;
  #pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * g + (r & 3);
      stage[row * D + ((32 * db + r32) ^ (((row >> 2) & 1) << 5))] = acc[db][r] * mul;
    }
  }
  // all chunks are read back before any is stored (the stores skip rows past the end,
  // and a read under that branch would wait on its own)
  constexpr int CH = D / 4, N = 32 * CH / 64;  // 16-byte chunks per row, per lane
  const int r0 = lane / CH, col = 4 * (lane % CH);
  f32x4 v[N];
  #pragma unroll
  for (int i = 0; i < N; ++i) {
    const int row = r0 + i * (64 / CH);
    v[i] = *reinterpret_cast<const f32x4*>(stage + row * D + (col ^ (((row >> 2) & 1) << 5)));
  }
  #pragma unroll
  for (int i = 0; i < N; ++i) sink.put(r0 + i * (64 / CH), col, v[i]);
}

// The mask's gradient (a learnable score bias) for one lane's 16 scores: dS = P (dP - Delta)
// of query row `row` at keys k0 + 8 rr + e (register 4 rr + e), added into dbias; by atomics
// where several heads or batch entries share the entries, else as 16-byte read-add-writes.
__device__ __forceinline__ void add_mask_grad(const BwdArgs& args, int b, int h, int row, int k0, const f32x16& ds) {
  const AttnShape& a = args.a;
  if (row >= a.Sq) return;
  float* db = args.dbias + b * args.dbias_sb + h * args.dbias_sh + (int64_t)row * args.dbias_sq;
  #pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int k4 = k0 + 8 * rr;
    if (!args.dbias_atomic && args.dbias_vec4 && k4 + 3 < a.Sk) {
      f32x4* p = reinterpret_cast<f32x4*>(db + k4);
      *p = *p + f32x4{ds[4 * rr], ds[4 * rr + 1], ds[4 * rr + 2], ds[4 * rr + 3]};
      continue;
    }
    #pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (k4 + e >= a.Sk) continue;
      if (args.dbias_atomic)
        __hip_atomic_fetch_add(db + k4 + e, ds[4 * rr + e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        db[k4 + e] += ds[4 * rr + e];
    }
  }
}

// Destination of a wave's 32-row result block: row 0's address and the row pitch in
// bytes, the rows that exist, and the element kind: bf16 (stored), fp32 (stored, a
// partial slice) or fp32 added to (an accumulator). Built once before the stores, so
// that a chunk's store is an address add and a store.
struct RowSink {
  char* base;
  int64_t pitch;
  int rows;
  int kind;  // 0 bf16, 1 fp32 store, 2 fp32 add
  __device__ __forceinline__ void put(int row, int col, const f32x4& v) const {
    if (row >= rows) return;
    char* p = base + row * pitch;
    if (kind == 0) {
      *reinterpret_cast<bf16x4*>(p + 2 * col) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    } else {
      f32x4* q = reinterpret_cast<f32x4*>(p + 4 * col);
      *q = kind == 2 ? *q + v : v;
    }
  }
};

// CAP: a logit softcap. The scores then leave the product raw: the cap's tanh sits between
// the product and the LSE, so the S half of the augmented k-chunk is not applied, and each
// slice reads -LSE / scale of its rows from the augmented rows in LDS. tanh(x) = 1 - 2 /
// (e^(2x) + 1) from the hardware exp2 and reciprocal, as in the forward; dS carries the
// cap's derivative 1 - tanh^2. Under additive scores (a dense mask's values or ALiBi, BIAS)
// the cap is applied to a whole block before they are added, with its derivative folded into
// dP - Delta; otherwise inside the woven slices.
// ST: the walk also stores each pair's dS (bf16, as the dK product takes it) into the pair's
// block of plan.ds, for a dQ pass that multiplies it by K instead of recomputing S and dP.
// NV: every pair is whole for the unit's keys (no causal diagonal or window, every key below
// the key length, no mask block other than open), so no score is masked per element: rows
// past the query length or the sequence end get P = 0 from their -inf statistic alone.
template <int D, bool CAUSAL, bool MASK, bool BIAS, bool CAP = false, int KVF = 0, bool ST = false, bool NV = false>
__device__ __forceinline__ void dkdv_unit(const BwdArgs& args, const BwdPlan& plan, int unit, char* smem) {
  constexpr int DS = D / 16, DB = D / 32;
  static_assert(8 % DS == 0 && 8 % (2 * DB) == 0, "each woven slice holds whole product pairs");
  using TL = Tile<D>;
  // three buffers: the pair being processed, the next one landing, and the one after it
  // staged as soon as this pair starts (the buffer it overwrites was last read two pairs
  // ago, before this pair's barrier)
  bf16* q_lds = reinterpret_cast<bf16*>(smem);                 // [3][KV_BM * D]
  bf16* do_lds = q_lds + 3 * KV_BM * D;                        // [3][KV_BM * D]
  // one extra 16-wide k-chunk per staged Q and dO row: (-LSE / scale) and (-Delta), each as
  // three bf16 terms (hi + mid + lo carry the fp32 value) and zeros; with K and V extended by
  // (1, 1, 1, 0 ...) the products give S - LSE / scale and dP - Delta directly, so the row
  // statistics are never broadcast to every lane through LDS
  bf16* aug_lds = do_lds + 3 * KV_BM * D;                      // [Q', dO'][3 buffers][KV_BM][16]

  const AttnShape& a = args.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) from here on
  const int g = lane >> 5, r32 = lane & 31;
  const KvUnit u = kv_unit_of(a, plan, unit);
  const int kt = u.kt, b = u.b, hk = u.hk, split = u.split;
  const int n0 = kt * KV_BN;
  const int key = n0 + 32 * wave + r32;
  const float cs = a.scale * kLog2e;
  const float cap_k = CAP ? 2.f * kLog2e * a.scale / a.softcap : 0.f, cap_raw = a.softcap * args.inv_scale;

  const bf16* K = static_cast<const bf16*>(args.k) + b * args.sk.b + hk * args.sk.h;
  const bf16* V = static_cast<const bf16*>(args.v) + b * args.sv.b + hk * args.sv.h;
  // (keys past the end read the last key: their scores are hidden on the tail tile and
  // their rows are never stored; a zeroing branch would make the loads wait here)
  const int64_t key_c = min(key, a.Sk - 1);
  // the K / V extension of the augmented chunk: (1, 1, 1, 0 ...) in half 0, zeros in half 1
  bf16x8 ones3;
  #pragma unroll
  for (int e = 0; e < 8; ++e) ones3[e] = (bf16)(g == 0 && e < 3 ? 1.f : 0.f);
  bf16x8 kf[DS], vf[DS];
  if constexpr (KVF == kKvBf16) {
    #pragma unroll
    for (int s = 0; s < DS; ++s) {
      kf[s] = *reinterpret_cast<const bf16x8*>(K + key_c * args.sk.s + 16 * s + 8 * g);
      vf[s] = *reinterpret_cast<const bf16x8*>(V + key_c * args.sv.s + 16 * s + 8 * g);
    }
  } else {  // a stored fp16 / q8_0 window: this lane's key row converted to bf16 in registers
    constexpr int KVE = KVF == kKvQ8 ? 1 : 2;
    const char* Kr = static_cast<const char*>(args.k) + (b * args.sk.b + hk * args.sk.h + key_c * args.sk.s) * KVE;
    const char* Vr = static_cast<const char*>(args.v) + (b * args.sv.b + hk * args.sv.h + key_c * args.sv.s) * KVE;
    const _Float16* Ks = a.kscale ? a.kscale + b * a.sks.b + hk * a.sks.h + key_c * a.sks.s : nullptr;
    const _Float16* Vs = a.vscale ? a.vscale + b * a.svs.b + hk * a.svs.h + key_c * a.svs.s : nullptr;
    #pragma unroll
    for (int s = 0; s < DS; ++s) {
      kf[s] = load_cvt8<KVF>(Kr, Ks, 16 * s + 8 * g);
      vf[s] = load_cvt8<KVF>(Vr, Vs, 16 * s + 8 * g);
    }
  }
  f32x16 dk[DB], dv[DB];
  #pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = zeros16();
    dv[db] = zeros16();
  }

  // the rows the structure lets see any of the unit's keys
  const int klen = klen_of(a, b), qlen = qlen_of(a, b);
  int qt0, qt_end;
  kv_row_tiles(a, klen, qlen, n0, qt0, qt_end);
  // the rows every key of the unit sees: a pair tile outside [r_lo, r_hi) needs masking
  // (as 32-bit row numbers: row bounds lie in [0, Sq])
  int r_lo, r_hi;
  {
    int64_t l0, h0, l1, h1;
    row_range(a, klen, qlen, n0, l0, h0);
    row_range(a, klen, qlen, n0 + KV_BN - 1, l1, h1);
    r_lo = (int)min<int64_t>(l1, a.Sq);
    r_hi = n0 + KV_BN > klen ? r_lo : (int)min<int64_t>(h0, a.Sq);  // keys past the length see nothing
  }
  // the (head, query tile) pairs this workgroup walks: query tiles qt0 .. qt_end - 1 of
  // every head of the group, pair p = (qt - qt0) * G + (h - hk G), p = split (mod kv_split)
  const int npairs = (qt_end - qt0) * a.G;

  // Pair p is (query tile qt0 + p / G, head hk G + p % G); this workgroup walks
  // p = split, split + kv_split, ..., carried as a running (quotient, remainder) so that
  // no step divides.
  struct Pos {
    int p, qi, hi, j;  // j: the candidate's number in this walk
  };
  const int step_q = plan.kv_split / a.G, step_h = plan.kv_split % a.G;
  auto advance = [&](Pos x) {
    x.p += plan.kv_split;
    ++x.j;
    x.qi += step_q;
    x.hi += step_h;
    if (x.hi >= a.G) {
      x.hi -= a.G;
      ++x.qi;
    }
    return x;
  };

  float lpre = 0.f;
  bool lrow = true;  // the staged statistic's row is below the query length
  // each of the first 2 KV_BM threads owns one augmented row in both buffers: zeroed once here
  // by the thread that later writes its three terms (so no barrier orders the two)
  if (tid < 2 * KV_BM) {
    #pragma unroll
    for (int bb = 0; bb < 3; ++bb) {
      bf16x8* z = reinterpret_cast<bf16x8*>(aug_lds + (((tid / KV_BM) * 3 + bb) * KV_BM + tid % KV_BM) * 16);
      zero(z[0]);
      zero(z[1]);
    }
  }
  auto pair_of = [&](const Pos& x, int& h, int& q0) {
    h = hk * a.G + x.hi;
    q0 = (qt0 + x.qi) * KV_BM;
  };
  // stage a pair's Q and dO tiles straight into LDS (rows past the end arrive as zeros,
  // masked out on the tail tile) and fetch its LSE / Delta into a register
  auto stage_pair = [&](const Pos& x, int buf) {
    int h, q0;
    pair_of(x, h, q0);
    const bf16* Q = static_cast<const bf16*>(args.q) + b * args.sq.b + h * args.sq.h + (int64_t)q0 * args.sq.s;
    const bf16* dO = static_cast<const bf16*>(args.dout) + b * args.sdo.b + h * args.sdo.h + (int64_t)q0 * args.sdo.s;
    TL::template stage_rows<KV_BM, NT>(q_lds + buf * KV_BM * D, Q, args.sq.s, a.Sq - q0);
    TL::template stage_rows<KV_BM, NT>(do_lds + buf * KV_BM * D, dO, args.sdo.s, a.Sq - q0);
    if (tid < 2 * KV_BM) {
      const int row = min(q0 + (tid % KV_BM), a.Sq - 1);
      // (turned into its three terms when stored, so that nothing waits for the load before
      // the tile's work)
      lpre = tid < KV_BM ? args.lse[b * args.lse_sb + h * args.lse_sh + row]
                         : args.delta[b * args.delta_sb + h * args.delta_sh + row];
      lrow = q0 + (tid % KV_BM) < qlen;
    }
  };
  // (a row past the query length or the sequence end gets -LSE / scale = -inf, as one term:
  // its scores are then -inf and P = 0 with or without the per-element masking)
  auto store_stats = [&](int buf) {
    if (tid < 2 * KV_BM) {
      const float c = tid < KV_BM ? (lrow ? -lpre * args.inv_scale : neg_inf()) : -lpre;
      const bf16 hi = (bf16)c;
      const bf16 mid = lrow || tid >= KV_BM ? (bf16)(c - (float)hi) : (bf16)0.f;
      const bf16 lo = lrow || tid >= KV_BM ? (bf16)(c - (float)hi - (float)mid) : (bf16)0.f;
      *reinterpret_cast<bf16x4*>(aug_lds + (((tid / KV_BM) * 3 + buf) * KV_BM + tid % KV_BM) * 16) =
          bf16x4{hi, mid, lo, (bf16)0.f};
    }
  };

  const int G16 = lane >> 4, L16 = lane & 15;
  const int tr_row = L16 >> 2, tr_col = 16 * (G16 & 1) + 4 * (L16 & 3);

  // With a mask tile map, pairs whose mask blocks are dead for both 64-key halves of
  // this workgroup are skipped; per wave, a dead block skips the products and an open
  // block skips the mask reads.
  const int nct = (a.Sk + kMaskTile - 1) / kMaskTile;
  const int ct0 = n0 / kMaskTile;
  auto live = [&](int j) -> bool {  // candidate j: pair split + j kv_split
    const int rt = qt0 + (split + j * plan.kv_split) / a.G;  // 64-row query tiles are the mask's row blocks
    for (int ct = ct0; ct < ct0 + KV_BN / kMaskTile && ct < nct; ++ct)
      if (tile_class(a, b, rt, ct) != kTileDead) return true;
    return false;
  };
  __shared__ uint64_t live_lds[kBwdWaves];
  LiveWords lw{live_lds, -NT, {0, 0, 0, 0}};
  const int ncand = npairs > split ? (npairs - split + plan.kv_split - 1) / plan.kv_split : 0;
  auto next_live = [&](Pos x) {
    if (!MASK || !a.tiles || x.p >= npairs) return x;
    const int j = lw.next(x.j, ncand, tid, live);
    if (j == x.j) return x;
    if (j >= ncand) return Pos{npairs, 0, 0, ncand};
    const int p = split + j * plan.kv_split;  // after a skip only
    return Pos{p, p / a.G, p % a.G, j};
  };
  const int ct_w = ct0 + (32 * wave) / kMaskTile;  // this wave's 32 keys lie in one 64-key block

  // Per-pair mask state of this wave, taken one pair ahead (its load completes under the
  // end-of-iteration wait instead of stalling the pair): the block class, from the wave's
  // run of classes down its key column (reloaded every 64 row blocks), and, for a 0 / -inf
  // block only, this lane's key column visibility word.
  const int nrt_all = (a.Sq + kMaskTile - 1) / kMaskTile;
  ClassRun run{kTileDead, -64};
  auto load_run = [&](int qi) {
    run.load(a, qi & ~63, ct_w < nct ? nrt_all - qt0 : 0,
             [&](int pos) { return tile_index(a, b, qt0 + pos, ct_w); });
  };
  auto mask_state = [&](const Pos& x, int& cls, uint64_t& w) {
    cls = kTileBias;
    w = ~0ull;
    if (MASK && a.tiles) {
      if (x.qi >= run.base + 64) load_run(x.qi);  // (a longer walk: the next 64 row blocks)
      cls = run.at(x.qi);
      if (cls == kTileBits)
        w = a.colbits[(int64_t)tile_index(a, b, qt0 + x.qi, ct_w) * kMaskTile + (key - ct_w * kMaskTile)];
    }
  };

  Pos cur = next_live(Pos{split, split / a.G, split % a.G, 0});
  int cls_cur = kTileBias;
  uint64_t wb_cur = ~0ull;
  if (cur.p < npairs) {
    stage_pair(cur, 0);
    if (MASK && a.tiles) {
      load_run(cur.qi);
      wait_vm();  // the run's classes, with the first pair's tiles
    }
    mask_state(cur, cls_cur, wb_cur);
  }
  // The K / V operand fragments live in accumulation registers for the whole walk (matrix
  // instructions read their A / B operands from there), leaving the vector file to the
  // pairs. Moved there only now, so that their loads and the first pair's land together.
  #pragma unroll
  for (int s = 0; s < DS; ++s) asm volatile("" : "+a"(kf[s]), "+a"(vf[s]));
  wait_vm();  // on every path: the K / V fragments are complete before the walk
  if (cur.p < npairs) store_stats(0);
  __syncthreads();
  // the first block's S / dP operands (Q, dO rows and their augmented chunks) of the pair
  // about to start, requested one pair ahead so that its products never wait on LDS
  bf16x8 pqa[DS], pda[DS], pqx, pdx;
  auto read_a0 = [&](int bb) {
    #pragma unroll
    for (int s = 0; s < DS; ++s) {
      pqa[s] = TL::read_chunk(q_lds + bb * KV_BM * D, r32, 2 * s + g);
      pda[s] = TL::read_chunk(do_lds + bb * KV_BM * D, r32, 2 * s + g);
    }
    pqx = *reinterpret_cast<const bf16x8*>(aug_lds + bb * KV_BM * 16 + r32 * 16 + 8 * g);
    pdx = *reinterpret_cast<const bf16x8*>(aug_lds + (3 + bb) * KV_BM * 16 + r32 * 16 + 8 * g);
  };
  if (cur.p < npairs) read_a0(0);
  // (ST) this lane's two 16-byte chunks of a 32-row block in the wave's 4 KB of a dS block:
  // chunk (block qb, half hh, key k, lane half g) at ((2 qb + hh) 32 + (k ^ 4 hh)) 2 + g.
  // Non-temporal stores: the blocks are read once, by the dQ pass, and not keeping them in
  // the caches leaves the next forward's operands there (whole LM step 2.5% faster).
  // Stored after the pair's wait, except under a softcap with additive scores, whose walk has
  // no registers to keep dS until then (stored as soon as formed)
  constexpr bool ST_LATE = !(CAP && BIAS);
  const uint32_t ds_off0 = (uint32_t)(r32 * 2 + g) * 16u, ds_off1 = 1024u + (uint32_t)((r32 ^ 4) * 2 + g) * 16u;
  for (int it = 0, buf = 0; cur.p < npairs; ++it) {
    const int nb = buf == 2 ? 0 : buf + 1;
    const Pos nxt = next_live(advance(cur));
    const bool more = nxt.p < npairs;
    int cls_next = kTileBias;
    uint64_t wb_next = ~0ull;
    if (more) {
      mask_state(nxt, cls_next, wb_next);
      stage_pair(nxt, nb);  // lands while this pair is being processed
    }
    int h, q0;
    pair_of(cur, h, q0);
    char* dsw = nullptr;  // (ST) the wave's 4 KB of this pair's dS block
    if constexpr (ST)
      dsw = plan.ds + ((((int64_t)b * a.Hq + h) * plan.ds_nku + kt) * plan.ds_nrt + q0 / KV_BM) * kDsBlock +
            wave * (kDsBlock / kBwdWaves);
    const int cls = cls_cur;
    const bool bias = MASK && (cls == kTileBias || a.alibi);  // add mask values and / or ALiBi
    const bool bits = MASK && cls == kTileBits;  // 0 / -inf block: use its visibility bits
    const bf16* qb_lds = q_lds + buf * KV_BM * D;
    const bf16* db_lds = do_lds + buf * KV_BM * D;
    const bf16* qx_lds = aug_lds + buf * KV_BM * 16;        // Q' rows of this pair
    const bf16* dx_lds = aug_lds + (3 + buf) * KV_BM * 16;  // dO' rows
    const bool edge = !(q0 >= r_lo && q0 + KV_BM <= r_hi);
    // Rows of the tile this lane's key can see, as a bit word (bit i: row q0 + i): the
    // structure (sequence ends, lengths, causal diagonal, window) and the block's
    // visibility bits (none for a dead block, whose products then contribute exact
    // zeros: skipping them per wave costs more in registers than it saves).
    const bool dead = MASK && cls == kTileDead;
    const bool masked = !NV && (edge || bits || dead);
    uint64_t vis = dead ? 0ull : ~0ull;
    if (masked && !dead) {
      int64_t lo, hi;
      row_range(a, klen, qlen, key, lo, hi);
      lo -= q0;
      hi -= q0;
      vis = bit_range64((int)(lo < 0 ? 0 : (lo > KV_BM ? KV_BM : lo)), (int)(hi < 0 ? 0 : (hi > KV_BM ? KV_BM : hi)));
      if (bits) vis &= wb_cur;
    }

    // The pair is two 32-row blocks, each in three steps: products S = Q K^T and
    // dP = dO V^T (A), the softmax gradient (B) and the products dV += P^T dO,
    // dK += dS^T Q (C). They run as A0, A1 with B0, C0 with B1, C1, so that each
    // block's vector work (B) has the other block's matrix products beside it; A0's
    // operands were requested before the previous pair's C1. Masking is applied
    // unconditionally (a no-op word on open blocks).
    // the augmented chunk of row 32 qb + r32 (half g: elements 8 g .. 8 g + 7)
    auto read_x = [&](const bf16* x_lds, int qb) {
      return *reinterpret_cast<const bf16x8*>(x_lds + (32 * qb + r32) * 16 + 8 * g);
    };
    // transpose reads of dO^T / Q^T for half hh of block qb (the operands of step C):
    // registers 8 hh .. 8 hh + 7 of the score accumulators hold rows
    // 32 qb + 16 hh + 8 t + 4 g + e, exactly the rows each read returns
    auto read_c = [&](int qb, int hh, bf16x8 (&dob)[DB], bf16x8 (&qbt)[DB]) {
      const int rbase = 32 * qb + 16 * hh + 4 * g + tr_row;
      #pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + tr_col;
        const bf16x4 d0 = TL::read_tr(db_lds, rbase, col);
        const bf16x4 d1 = TL::read_tr(db_lds, rbase + 8, col);
        const bf16x4 q0v = TL::read_tr(qb_lds, rbase, col);
        const bf16x4 q1v = TL::read_tr(qb_lds, rbase + 8, col);
        dob[db] = bf16x8{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        qbt[db] = bf16x8{q0v[0], q0v[1], q0v[2], q0v[3], q1v[0], q1v[1], q1v[2], q1v[3]};
      }
    };
    auto step_c = [&](int qb, const bf16x8 (&pa)[2], const bf16x8 (&dsa)[2]) {
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 dob[DB], qbt[DB];
        read_c(qb, hh, dob, qbt);
        #pragma unroll
        for (int db = 0; db < DB; ++db) {
          mma_acc(dv[db], pa[hh], dob[db]);
          mma_acc(dk[db], dsa[hh], qbt[db]);
        }
      }
    };
    // step B for block qb, scores in sacc / dpacc (lane = key, half g; register r = query
    // row 32 qb + 8 (r/4) + 4 g + r%4): additive mask values and the row statistics
    // first, then slice i finishes registers 2 i and 2 i + 1 (hidden scores -> -inf,
    // P = 0; bit 8 rr + e of the visibility word <-> register 4 rr + e)
    struct RowStats {
      uint32_t w;
      const bf16* x;  // (CAP) the augmented row of register 0's query row
    };
    auto stats_b = [&](int qb, f32x16& sacc, f32x16& dpacc, RowStats& st) {
      if constexpr (CAP && BIAS) {
        // a softcap under additive scores: the cap goes first (the mask and ALiBi add to the
        // capped score), its derivative 1 - tanh^2 joins dP - Delta here, and the slices then
        // only add -LSE / scale
        #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float t = 1.f - 2.f * __builtin_amdgcn_rcpf(fast_exp2(sacc[r] * cap_k) + 1.f);
          sacc[r] = cap_raw * t;
          dpacc[r] *= 1.f - t * t;
          if (r % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // (a few registers in flight at a time)
        }
      }
      if (BIAS && bias && a.alibi) {
        // ALiBi in raw score units: -(slope / scale) |key - position|; this lane's key, the
        // register's row: key - position = (key - q_offset - q0 - 32 qb - 4 g) - 8 (r/4) - r%4
        const float sl = a.alibi[h] * args.inv_scale;
        const float base = (float)((int64_t)key - a.q_offset - q0 - 32 * qb - 4 * g);
        #pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] -= sl * fabsf(base - (float)(8 * (r >> 2) + (r & 3)));
      }
      if (BIAS && bias && a.mask) {
        const float* mk = a.mask + b * a.mask_sb + h * a.mask_sh + min(key, a.Sk - 1);
        #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = min(q0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3), a.Sq - 1);
          sacc[r] += mk[(int64_t)row * a.mask_sq] * args.inv_scale;
        }
      }
      st.w = (uint32_t)(vis >> (32 * qb + 4 * g));
      st.x = qx_lds + (32 * qb + 4 * g) * 16;
    };
    auto slice_b = [&](int i, const RowStats& st, f32x16& sacc, f32x16& dpacc) {
      if constexpr (CAP && BIAS) {  // (capped, with the additive values and the derivative, in stats_b)
        #pragma unroll
        for (int r = 2 * i; r < 2 * i + 2; ++r) {
          const bf16x4 c3 = *reinterpret_cast<const bf16x4*>(st.x + (8 * (r >> 2) + (r & 3)) * 16);
          const float nl = (float)c3[0] + (float)c3[1] + (float)c3[2];
          const float sv = ninf_unless_bit(sacc[r] + nl, st.w, 8 * (r >> 2) + (r & 3));
          const float pv = fast_exp2(sv * cs);
          sacc[r] = pv;
          dpacc[r] = pv * dpacc[r];
        }
        return;
      }
      if constexpr (CAP) {
        #pragma unroll
        for (int r = 2 * i; r < 2 * i + 2; ++r) {
          // -LSE / scale of the register's row: the three terms of its augmented row
          const bf16x4 c3 = *reinterpret_cast<const bf16x4*>(st.x + (8 * (r >> 2) + (r & 3)) * 16);
          const float nl = (float)c3[0] + (float)c3[1] + (float)c3[2];
          const float t = 1.f - 2.f * __builtin_amdgcn_rcpf(fast_exp2(sacc[r] * cap_k) + 1.f);
          const float sv = ninf_unless_bit(fmaf(cap_raw, t, nl), st.w, 8 * (r >> 2) + (r & 3));
          const float pv = fast_exp2(sv * cs);
          sacc[r] = pv;
          dpacc[r] = pv * dpacc[r] * (1.f - t * t);
        }
        return;
      }
      #pragma unroll
      for (int r = 2 * i; r < 2 * i + 2; ++r) {
        // (the products already hold S - LSE / scale and dP - Delta)
        const float sv = NV ? sacc[r] : ninf_unless_bit(sacc[r], st.w, 8 * (r >> 2) + (r & 3));
        const float pv = fast_exp2(sv * cs);
        sacc[r] = pv;
        dpacc[r] = pv * dpacc[r];
      }
    };
    f32x16 s0, dp0, s1, dp1;
    bf16x8 pa0[2], ds0[2], pa1[2], ds1[2];
    s0 = zeros16();  // step A of block 0 from the operands requested one pair ahead
    dp0 = zeros16();
    #pragma unroll
    for (int s = 0; s < DS; ++s) {
      mma(s0, pqa[s], kf[s]);
      mma(dp0, pda[s], vf[s]);
    }
    if constexpr (!CAP) mma(s0, pqx, ones3);
    mma(dp0, pdx, ones3);
    // Step A of block 1 woven with step B of block 0, then step C of block 0 woven with
    // step B of block 1: each two are independent, and one wave per SIMD only overlaps
    // vector work with matrix products when its instruction stream alternates them. Each
    // slice is two products and two scores, fenced so that the scheduler keeps the
    // alternation; the operands of both are loaded before the weave.
    {
      bf16x8 qa[DS], da[DS];
      #pragma unroll
      for (int s = 0; s < DS; ++s) {
        qa[s] = TL::read_chunk(qb_lds, 32 + r32, 2 * s + g);
        da[s] = TL::read_chunk(db_lds, 32 + r32, 2 * s + g);
      }
      const bf16x8 qx = read_x(qx_lds, 1), dx = read_x(dx_lds, 1);
      RowStats st;
      stats_b(0, s0, dp0, st);
      s1 = zeros16();
      dp1 = zeros16();
      __builtin_amdgcn_sched_barrier(0);
      // DS product pairs spread over the 8 slices, the augmented pair in the last
      #pragma unroll
      for (int i = 0; i < 8; ++i) {
        constexpr int EVERY = 8 / DS;
        if (i % EVERY == 0) {
          mma(s1, qa[i / EVERY], kf[i / EVERY]);
          mma(dp1, da[i / EVERY], vf[i / EVERY]);
        }
        if (i == 7) {
          if constexpr (!CAP) mma(s1, qx, ones3);
          mma(dp1, dx, ones3);
        }
        slice_b(i, st, s0, dp0);
        __builtin_amdgcn_sched_barrier(0);
      }
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        pack8(pa0[hh], s0, 8 * hh);
        pack8(ds0[hh], dp0, 8 * hh);
      }
      if constexpr (ST && !ST_LATE) {
        __builtin_nontemporal_store(ds0[0], reinterpret_cast<bf16x8*>(dsw + ds_off0));
        __builtin_nontemporal_store(ds0[1], reinterpret_cast<bf16x8*>(dsw + ds_off1));
      }
    }
    {
      bf16x8 dob[2][DB], qbt[2][DB];
      read_c(0, 0, dob[0], qbt[0]);
      read_c(0, 1, dob[1], qbt[1]);
      RowStats st;
      stats_b(1, s1, dp1, st);
      __builtin_amdgcn_sched_barrier(0);
      // 2 DB product pairs spread over the 8 slices
      #pragma unroll
      for (int i = 0; i < 8; ++i) {
        constexpr int EVERY = 8 / (2 * DB);
        if (i % EVERY == 0) {
          const int j = i / EVERY, hh = j / DB, db = j % DB;
          mma_acc(dv[db], pa0[hh], dob[hh][db]);
          mma_acc(dk[db], ds0[hh], qbt[hh][db]);
        }
        slice_b(i, st, s1, dp1);
        __builtin_amdgcn_sched_barrier(0);
      }
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        pack8(pa1[hh], s1, 8 * hh);
        pack8(ds1[hh], dp1, 8 * hh);
      }
      if constexpr (ST && !ST_LATE) {
        __builtin_nontemporal_store(ds1[0], reinterpret_cast<bf16x8*>(dsw + 2048 + ds_off0));
        __builtin_nontemporal_store(ds1[1], reinterpret_cast<bf16x8*>(dsw + 2048 + ds_off1));
      }
    }
    // the next pair's tiles are complete once every wave has waited for its own loads;
    // its first block's operands are then requested before this pair's last products
    wait_vm();
    if (more) store_stats(nb);
    __syncthreads();
    if (more) read_a0(nb);
    step_c(1, pa1, ds1);
    if constexpr (ST && ST_LATE) {
      // (after this pair's wait: the stores complete under the next pair, whose end-of-pair
      // wait would otherwise also wait for them)
      __builtin_nontemporal_store(ds0[0], reinterpret_cast<bf16x8*>(dsw + ds_off0));
      __builtin_nontemporal_store(ds0[1], reinterpret_cast<bf16x8*>(dsw + ds_off1));
      __builtin_nontemporal_store(ds1[0], reinterpret_cast<bf16x8*>(dsw + 2048 + ds_off0));
      __builtin_nontemporal_store(ds1[1], reinterpret_cast<bf16x8*>(dsw + 2048 + ds_off1));
    }
    buf = nb;
    cur = nxt;
    cls_cur = cls_next;
    wb_cur = wb_next;
  }

  settle_acc(dk);
  settle_acc(dv);
  // Split walks store their partial sums (unscaled) into their own fp32 slice, which a
  // reduce pass sums; a workgroup with no live pair still stores its zeros. The pair
  // buffers stage the results once every wave has left the walk.
  const bool part = plan.kv_split > 1;
  const int kbase = n0 + 32 * wave;
  const int rows = max(0, min(32, a.Sk - kbase));
  auto sink = [&](float* part_base, void* out, const Strides& so) {
    if (part)
      return RowSink{reinterpret_cast<char*>(part_base + (int64_t)split * a.B * a.Hkv * a.Sk * D +
                                             (((int64_t)b * a.Hkv + hk) * a.Sk + kbase) * D),
                     (int64_t)D * 4, rows, 1};
    const int64_t esz = args.accumulate ? 4 : 2;
    return RowSink{static_cast<char*>(out) + (b * so.b + hk * so.h + (int64_t)kbase * so.s) * esz, so.s * esz, rows,
                   args.accumulate ? 2 : 0};
  };
  const RowSink sk = sink(plan.dk_part, args.dk, args.sdk), sv = sink(plan.dv_part, args.dv, args.sdv);
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * D;
  __syncthreads();
  store_block<D>(dk, part ? 1.f : a.scale, stage, lane, sk);
  store_block<D>(dv, 1.f, stage, lane, sv);
}

// ---------------------------------------------------------------------------
// dK / dV workgroup with the work split by role (two workgroups per compute unit)
// ---------------------------------------------------------------------------
// A 64-key tile of one KV head, walked by four waves: for each 32-key group, one wave
// computes S = Q K^T, P and dV += P^T dO (role 0) and another dP = dO V^T, dS and
// dK += dS^T Q (role 1). Each wave holds one operand (K or V) and one accumulator (dV or
// dK) of its 32 keys, about half the registers of a wave doing all four products, so
// two workgroups share a compute unit and each one's waits are covered by the other's
// products. P reaches the dS wave through LDS in bf16, in the accumulator layout both
// waves share (lane = key, register = query row), 2 KB per block; dS is then formed from
// it (one more bf16 rounding of P inside the products, as dV already uses it). Per
// (head, 64-row query tile) pair:
//   role 0: S0, P0 -> LDS; S1, P1 -> LDS | barrier | dV += P0^T dO0, P1^T dO1
//   role 1: dP0, dP1                     | barrier | dS0 -> dK += dS0^T Q0; dS1 -> dK
// The structure, the mask's block classes and visibility bits, its additive values and
// ALiBi are applied by role 0 (P = 0 exactly where hidden, so role 1's dS is 0 there).
// The rest is the one-wave walk's: pairs of a split walk, the live-candidate words, the
// Q / dO tiles copied straight into LDS one pair ahead (two buffers), LSE and Delta
// folded into an extra k-chunk of the products, results stored through LDS.
template <int D, bool CAUSAL, bool MASK, bool BIAS>
__device__ __forceinline__ void dkdv_role_unit(const BwdArgs& args, const BwdPlan& plan, int unit, char* smem) {
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int BN = kBwdRoleKeys, BM = KV_BM;
  using TL = Tile<D>;
  bf16* q_lds = reinterpret_cast<bf16*>(smem);     // [2][BM * D]
  bf16* do_lds = q_lds + 2 * BM * D;               // [2][BM * D]
  // augmented k-chunk rows: (-LSE / scale) and (-Delta) as three bf16 terms (hi + mid + lo
  // carry the fp32 value), 8 elements per row; both lane halves read them and the K / V
  // extension (1, 1, 1, 0 ...) is zero in half 1, so only half 0's copy counts
  bf16* aug_lds = do_lds + 2 * BM * D;             // [Q', dO'][2 buffers][BM][8]
  bf16* x_lds = aug_lds + 2 * 2 * BM * 8;          // P exchange [2 blocks][2 key groups][64 lanes][16]

  const AttnShape& a = args.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave >> 1, kg = wave & 1;  // role 0: S, P, dV; role 1: dP, dS, dK
  const int g = lane >> 5, r32 = lane & 31;
  const KvUnit u = kv_unit_of(a, plan, unit);
  const int kt = u.kt, b = u.b, hk = u.hk, split = u.split;
  const int n0 = kt * BN;
  const int key = n0 + 32 * kg + r32;
  const float cs = a.scale * kLog2e;

  // this wave's operand: K (role 0) or V (role 1), rows of its 32 keys (keys past the end
  // read the last key: their scores are hidden on the tail tile, their rows never stored)
  const bf16* KV = role == 0 ? static_cast<const bf16*>(args.k) + b * args.sk.b + hk * args.sk.h
                             : static_cast<const bf16*>(args.v) + b * args.sv.b + hk * args.sv.h;
  const int64_t kv_s = role == 0 ? args.sk.s : args.sv.s;
  const int64_t key_c = min(key, a.Sk - 1);
  bf16x8 ones3;
  #pragma unroll
  for (int e = 0; e < 8; ++e) ones3[e] = (bf16)(g == 0 && e < 3 ? 1.f : 0.f);
  bf16x8 kvf[DS];
  #pragma unroll
  for (int s = 0; s < DS; ++s) kvf[s] = *reinterpret_cast<const bf16x8*>(KV + key_c * kv_s + 16 * s + 8 * g);
  f32x16 acc[DB];  // dV (role 0) or dK (role 1)
  #pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zeros16();

  // the rows that can see any of the unit's keys, and the rows every key sees (a pair
  // tile outside [r_lo, r_hi) needs masking), as in the one-wave walk
  const int klen = klen_of(a, b), qlen = qlen_of(a, b);
  int qt0 = 0, qt_end = 0;
  if (n0 < klen) {
    int64_t lo, hi, lo1, hi1;
    row_range(a, klen, qlen, n0, lo, hi);
    row_range(a, klen, qlen, min(n0 + BN, klen) - 1, lo1, hi1);
    const int nqt = (a.Sq + BM - 1) / BM;
    qt0 = (int)min<int64_t>(lo / BM, nqt);
    qt_end = hi1 > lo ? (int)min<int64_t>((hi1 + BM - 1) / BM, nqt) : qt0;
    if (qt_end < qt0) qt_end = qt0;
  }
  int r_lo, r_hi;
  {
    int64_t l0, h0, l1, h1;
    row_range(a, klen, qlen, n0, l0, h0);
    row_range(a, klen, qlen, n0 + BN - 1, l1, h1);
    r_lo = (int)min<int64_t>(l1, a.Sq);
    r_hi = n0 + BN > klen ? r_lo : (int)min<int64_t>(h0, a.Sq);
  }
  const int npairs = (qt_end - qt0) * a.G;
  struct Pos {
    int p, qi, hi, j;
  };
  const int step_q = plan.kv_split / a.G, step_h = plan.kv_split % a.G;
  auto advance = [&](Pos x) {
    x.p += plan.kv_split;
    ++x.j;
    x.qi += step_q;
    x.hi += step_h;
    if (x.hi >= a.G) {
      x.hi -= a.G;
      ++x.qi;
    }
    return x;
  };
  auto pair_of = [&](const Pos& x, int& h, int& q0) {
    h = hk * a.G + x.hi;
    q0 = (qt0 + x.qi) * BM;
  };
  float lpre = 0.f;
  auto stage_pair = [&](const Pos& x, int buf) {
    int h, q0;
    pair_of(x, h, q0);
    const bf16* Q = static_cast<const bf16*>(args.q) + b * args.sq.b + h * args.sq.h + (int64_t)q0 * args.sq.s;
    const bf16* dO = static_cast<const bf16*>(args.dout) + b * args.sdo.b + h * args.sdo.h + (int64_t)q0 * args.sdo.s;
    TL::template stage<BM, NT, false>(q_lds + buf * BM * D, Q, args.sq.s, a.Sq - q0);
    TL::template stage<BM, NT, false>(do_lds + buf * BM * D, dO, args.sdo.s, a.Sq - q0);
    if (tid < 2 * BM) {
      const int row = min(q0 + (tid % BM), a.Sq - 1);
      lpre = tid < BM ? args.lse[b * args.lse_sb + h * args.lse_sh + row]
                      : args.delta[b * args.delta_sb + h * args.delta_sh + row];
    }
  };
  auto store_stats = [&](int buf) {
    if (tid < 2 * BM) {
      const float c = tid < BM ? -lpre * args.inv_scale : -lpre;
      const bf16 hi = (bf16)c;
      const bf16 mid = (bf16)(c - (float)hi);
      const bf16 lo = (bf16)(c - (float)hi - (float)mid);
      *reinterpret_cast<bf16x8*>(aug_lds + (((tid / BM) * 2 + buf) * BM + tid % BM) * 8) =
          bf16x8{hi, mid, lo, (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    }
  };

  const int G16 = lane >> 4, L16 = lane & 15;
  const int tr_row = L16 >> 2, tr_col = 16 * (G16 & 1) + 4 * (L16 & 3);

  // pairs whose mask block is dead are skipped by the whole workgroup; per pair, role 0
  // takes the block class and, for a 0 / -inf block, its key's visibility word
  const int nct = (a.Sk + kMaskTile - 1) / kMaskTile;
  const int ct0 = n0 / kMaskTile;  // the unit's keys are one mask block column
  auto live = [&](int j) -> bool {
    const int rt = qt0 + (split + j * plan.kv_split) / a.G;
    return ct0 < nct && tile_class(a, b, rt, ct0) != kTileDead;
  };
  __shared__ uint64_t live_lds[kBwdWaves];
  LiveWords lw{live_lds, -NT, {0, 0, 0, 0}};
  const int ncand = npairs > split ? (npairs - split + plan.kv_split - 1) / plan.kv_split : 0;
  auto next_live = [&](Pos x) {
    if (!MASK || !a.tiles || x.p >= npairs) return x;
    const int j = lw.next(x.j, ncand, tid, live);
    if (j == x.j) return x;
    if (j >= ncand) return Pos{npairs, 0, 0, ncand};
    const int p = split + j * plan.kv_split;
    return Pos{p, p / a.G, p % a.G, j};
  };
  const int nrt_all = (a.Sq + kMaskTile - 1) / kMaskTile;
  ClassRun run{kTileDead, -64};
  auto load_run = [&](int qi) {
    run.load(a, qi & ~63, ct0 < nct ? nrt_all - qt0 : 0, [&](int pos) { return tile_index(a, b, qt0 + pos, ct0); });
  };
  auto mask_state = [&](const Pos& x, int& cls, uint64_t& w) {
    cls = kTileBias;
    w = ~0ull;
    if (MASK && a.tiles) {
      if (x.qi >= run.base + 64) load_run(x.qi);
      cls = run.at(x.qi);
      if (cls == kTileBits)
        w = a.colbits[(int64_t)tile_index(a, b, qt0 + x.qi, ct0) * kMaskTile + (key - ct0 * kMaskTile)];
    }
  };

  Pos cur = next_live(Pos{split, split / a.G, split % a.G, 0});
  int cls_cur = kTileBias;
  uint64_t wb_cur = ~0ull;
  if (cur.p < npairs) {
    stage_pair(cur, 0);
    if (MASK && a.tiles) {
      load_run(cur.qi);
      wait_vm();
    }
    mask_state(cur, cls_cur, wb_cur);
  }
  // (everything stays in the arch VGPRs: about 200 per lane, so that with no AGPRs in use the
  // compiler may give this walk all 256 registers of a two-workgroups-per-unit wave)
  wait_vm();
  if (cur.p < npairs) store_stats(0);
  __syncthreads();
  bf16* xw = x_lds + (kg * 64 + lane) * 16;  // this lane's P slot, block 0 (block 1: + 2 * 64 * 16)

  // the pair loop, compiled once per role so that each wave's loop carries only its own
  // role's operands and addresses (both loops take the same barriers in the same order)
  auto walk = [&](auto role_c) {
  constexpr int ROLE = decltype(role_c)::value;
  for (int buf = 0; cur.p < npairs;) {
    const int nb = buf ^ 1;
    const Pos nxt = next_live(advance(cur));
    const bool more = nxt.p < npairs;
    int cls_next = kTileBias;
    uint64_t wb_next = ~0ull;
    if (more) {
      mask_state(nxt, cls_next, wb_next);
      stage_pair(nxt, nb);  // lands while this pair is processed
    }
    int h, q0;
    pair_of(cur, h, q0);
    const bf16* qb_lds = q_lds + buf * BM * D;
    const bf16* db_lds = do_lds + buf * BM * D;
    // Three phases per pair, separated by workgroup barriers, each with about the same
    // matrix work for both roles (role 0 | role 1):
    //   S0, P0 -> LDS          | dP0
    //   dV += P0^T dO0; S1, P1 | dS0 (P0 from LDS), dK += dS0^T Q0; dP1
    //   dV += P1^T dO1         | dS1, dK += dS1^T Q1
    if constexpr (ROLE == 0) {
      const int cls = cls_cur;
      const bool bias = BIAS && MASK && (cls == kTileBias || a.alibi);
      const bool bits = MASK && cls == kTileBits;
      const bool dead = MASK && cls == kTileDead;
      const bool edge = !(q0 >= r_lo && q0 + BM <= r_hi);
      const bool masked = edge || bits || dead;
      uint64_t vis = dead ? 0ull : ~0ull;
      if (masked && !dead) {
        int64_t lo, hi;
        row_range(a, klen, qlen, key, lo, hi);
        lo -= q0;
        hi -= q0;
        vis = bit_range64((int)(lo < 0 ? 0 : (lo > BM ? BM : lo)), (int)(hi < 0 ? 0 : (hi > BM ? BM : hi)));
        if (bits) vis &= wb_cur;
      }
      const bf16* qx_lds = aug_lds + buf * BM * 8;
      // S and P of block qb (lane = key, half g; register r = query row 32 qb + 8 (r/4) + 4 g + r%4),
      // stored to this lane's P slot and kept for dV
      auto s_block = [&](int qb, bf16x8 (&pa)[2]) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 qa[DS];
        #pragma unroll
        for (int s = 0; s < DS; ++s) qa[s] = TL::read_chunk(qb_lds, 32 * qb + r32, 2 * s + g);
        const bf16x8 qx = *reinterpret_cast<const bf16x8*>(qx_lds + (32 * qb + r32) * 8);
        f32x16 sacc = zeros16();
        #pragma unroll
        for (int s = 0; s < DS; ++s) mma(sacc, qa[s], kvf[s]);
        mma(sacc, qx, ones3);  // S - LSE / scale
        if (bias && a.alibi) {
          const float sl = a.alibi[h] * args.inv_scale;
          const float base = (float)((int64_t)key - a.q_offset - q0 - 32 * qb - 4 * g);
          #pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] -= sl * fabsf(base - (float)(8 * (r >> 2) + (r & 3)));
        }
        if (bias && a.mask) {  // four rows' values in flight at a time (registers)
          const float* mk = a.mask + b * a.mask_sb + h * a.mask_sh + min(key, a.Sk - 1);
          #pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            float mv[4];
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int row = min(q0 + 32 * qb + 8 * rr + 4 * g + e, a.Sq - 1);
              mv[e] = mk[(int64_t)row * a.mask_sq];
            }
            #pragma unroll
            for (int e = 0; e < 4; ++e) sacc[4 * rr + e] += mv[e] * args.inv_scale;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (masked) {  // hidden scores -> -inf (P = 0); bit 8 rr + e of w <-> register 4 rr + e
          const uint32_t w = (uint32_t)(vis >> (32 * qb + 4 * g));
          #pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = ninf_unless_bit(sacc[r], w, 8 * (r >> 2) + (r & 3));
        }
        #pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(sacc[r] * cs);
        pack8(pa[0], sacc, 0);
        pack8(pa[1], sacc, 8);
        *reinterpret_cast<bf16x8*>(xw + qb * 2 * 64 * 16) = pa[0];
        *reinterpret_cast<bf16x8*>(xw + qb * 2 * 64 * 16 + 8) = pa[1];
      };
      // dV += P^T dO for block qb: registers 8 hh .. of P hold rows 32 qb + 16 hh + 8 t + 4 g + e,
      // the rows each pair of dO^T transpose reads returns
      // (the reads of one half, 8 transposes, are issued before its 4 products and fenced from
      // the other half's, so that at most 16 operand registers are in flight)
      auto dv_block = [&](int qb, const bf16x8 (&pa)[2]) {
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int rbase = 32 * qb + 16 * hh + 4 * g + tr_row;
          bf16x8 dob[DB];
          #pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x4 d0 = TL::read_tr(db_lds, rbase, 32 * db + tr_col);
            const bf16x4 d1 = TL::read_tr(db_lds, rbase + 8, 32 * db + tr_col);
            dob[db] = bf16x8{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
          }
          #pragma unroll
          for (int db = 0; db < DB; ++db) mma(acc[db], pa[hh], dob[db]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      bf16x8 p0[2], p1[2];
      s_block(0, p0);
      __syncthreads();
      dv_block(0, p0);
      s_block(1, p1);
      __syncthreads();
      dv_block(1, p1);
    } else {
      const bf16* dx_lds = aug_lds + (2 + buf) * BM * 8;
      auto dp_block = [&](int qb) {  // dP - Delta of block qb
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 da[DS];
        #pragma unroll
        for (int s = 0; s < DS; ++s) da[s] = TL::read_chunk(db_lds, 32 * qb + r32, 2 * s + g);
        const bf16x8 dx = *reinterpret_cast<const bf16x8*>(dx_lds + (32 * qb + r32) * 8);
        f32x16 dp = zeros16();
        #pragma unroll
        for (int s = 0; s < DS; ++s) mma(dp, da[s], kvf[s]);
        mma(dp, dx, ones3);
        return dp;
      };
      // dS = P (dP - Delta) from role 0's P of block qb, then dK += dS^T Q
      auto dk_block = [&](int qb, f32x16& dp) {
        const bf16x8 pv0 = *reinterpret_cast<const bf16x8*>(xw + qb * 2 * 64 * 16);
        const bf16x8 pv1 = *reinterpret_cast<const bf16x8*>(xw + qb * 2 * 64 * 16 + 8);
        #pragma unroll
        for (int r = 0; r < 8; ++r) {
          dp[r] *= (float)pv0[r];
          dp[8 + r] *= (float)pv1[r];
        }
        bf16x8 dsa[2];
        pack8(dsa[0], dp, 0);
        pack8(dsa[1], dp, 8);
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int rbase = 32 * qb + 16 * hh + 4 * g + tr_row;
          bf16x8 qbt[DB];
          #pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x4 q0v = TL::read_tr(qb_lds, rbase, 32 * db + tr_col);
            const bf16x4 q1v = TL::read_tr(qb_lds, rbase + 8, 32 * db + tr_col);
            qbt[db] = bf16x8{q0v[0], q0v[1], q0v[2], q0v[3], q1v[0], q1v[1], q1v[2], q1v[3]};
          }
          #pragma unroll
          for (int db = 0; db < DB; ++db) mma(acc[db], dsa[hh], qbt[db]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      f32x16 dp0 = dp_block(0);
      __syncthreads();  // role 0 has stored P0
      dk_block(0, dp0);
      f32x16 dp1 = dp_block(1);
      __syncthreads();  // role 0 has stored P1
      dk_block(1, dp1);
    }
    // the next pair's tiles are complete once every wave has waited for its own loads;
    // every read of this pair's buffers and P slots is done after this barrier
    wait_vm();
    if (more) store_stats(nb);
    __syncthreads();
    buf = nb;
    cur = nxt;
    cls_cur = cls_next;
    wb_cur = wb_next;
  }
  };
  if (role == 0)
    walk(std::integral_constant<int, 0>{});
  else
    walk(std::integral_constant<int, 1>{});

  const bool part = plan.kv_split > 1;
  const int kbase = n0 + 32 * kg;
  const int rows = max(0, min(32, a.Sk - kbase));
  float* part_base = role == 0 ? plan.dv_part : plan.dk_part;
  void* out = role == 0 ? args.dv : args.dk;
  const Strides so = role == 0 ? args.sdv : args.sdk;
  RowSink sink;
  if (part) {
    sink = RowSink{reinterpret_cast<char*>(part_base + (int64_t)split * a.B * a.Hkv * a.Sk * D +
                                           (((int64_t)b * a.Hkv + hk) * a.Sk + kbase) * D),
                   (int64_t)D * 4, rows, 1};
  } else {
    const int64_t esz = args.accumulate ? 4 : 2;
    sink = RowSink{static_cast<char*>(out) + (b * so.b + hk * so.h + (int64_t)kbase * so.s) * esz, so.s * esz, rows,
                   args.accumulate ? 2 : 0};
  }
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * D;
  __syncthreads();
  store_block<D>(acc, (role == 1 && !part) ? a.scale : 1.f, stage, lane, sink);
}

// ---------------------------------------------------------------------------
// dQ workgroup
// ---------------------------------------------------------------------------
// MG: the mask's gradient is requested (a masked, uncapped problem; kernels of their own, so that
// the others carry none of its code)
template <int D, bool CAUSAL, bool MASK, bool BIAS, bool LOWREG = false, bool CAP = false, int KVF = 0, bool MG = false>
__device__ __forceinline__ void dq_unit(const BwdArgs& args, const BwdPlan& plan, int unit, char* smem) {
  constexpr int DS = D / 16, DB = D / 32;
  using TL = Tile<D>;
  bf16* k_lds = reinterpret_cast<bf16*>(smem);  // [2][Q_BN * D]
  bf16* v_lds = k_lds + 2 * Q_BN * D;           // [2][Q_BN * D]

  const AttnShape& a = args.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) from here on
  const int g = lane >> 5, r32 = lane & 31;
  const QUnit u = q_unit_of(a, plan, unit);
  const int qt = u.qt, b = u.b, h = u.h, split = u.split, nsplit = u.nsplit;
  const int hk = h / a.G;
  const int q0 = qt * Q_BM;
  const int qw = q0 + 32 * wave;
  const int row = qw + r32;
  const float cs = a.scale * kLog2e;
  const float cap_k = CAP ? 2.f * kLog2e * a.scale / a.softcap : 0.f, cap_raw = a.softcap * args.inv_scale;

  const bf16* Q = static_cast<const bf16*>(args.q) + b * args.sq.b + h * args.sq.h;
  const bf16* dO = static_cast<const bf16*>(args.dout) + b * args.sdo.b + h * args.sdo.h;
  const bf16* K = static_cast<const bf16*>(args.k) + b * args.sk.b + hk * args.sk.h;
  const bf16* V = static_cast<const bf16*>(args.v) + b * args.sv.b + hk * args.sv.h;
  // (rows past the end read the last row: their scores are hidden on the tail tile and
  // their dQ rows are never stored; a zeroing branch would make the loads wait here)
  const int64_t row_c = min(row, a.Sq - 1);
  bf16x8 qf[DS], df[DS];
  #pragma unroll
  for (int s = 0; s < DS; ++s) {
    qf[s] = *reinterpret_cast<const bf16x8*>(Q + row_c * args.sq.s + 16 * s + 8 * g);
    df[s] = *reinterpret_cast<const bf16x8*>(dO + row_c * args.sdo.s + 16 * s + 8 * g);
  }
  const float lse2 = args.lse[b * args.lse_sb + h * args.lse_sh + row_c] * kLog2e;
  const float dlt = args.delta[b * args.delta_sb + h * args.delta_sh + row_c];
  if constexpr (LOWREG) {
    // two workgroups per compute unit: the Q / dO fragments wait in accumulation
    // registers (matrix instructions read their operands there), leaving the vector
    // file to the walk
    #pragma unroll
    for (int s = 0; s < DS; ++s) asm volatile("" : "+a"(qf[s]), "+a"(df[s]));
  }

  f32x16 dq[DB];
  #pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = zeros16();

  // keys the workgroup's rows can see by the structure (sequence ends, causal diagonal,
  // key and query lengths, window): from the first row's lower end to the last visible
  // row's upper end (both ends move right with the row)
  const int klen = klen_of(a, b), qlen = qlen_of(a, b);
  const int nkt = (a.Sk + Q_BN - 1) / Q_BN;
  int kt_begin = 0, kt_end = 0;
  if (q0 < qlen) {
    int64_t lo, hi, lo1, hi1;
    key_range(a, klen, qlen, q0, lo, hi);
    key_range(a, klen, qlen, min(q0 + Q_BM, qlen) - 1, lo1, hi1);
    kt_begin = (int)min<int64_t>(lo / Q_BN, nkt);
    kt_end = hi1 > lo ? (int)min<int64_t>((hi1 + Q_BN - 1) / Q_BN, nkt) : kt_begin;
    if (kt_end < kt_begin) kt_end = kt_begin;
  }
  // the keys every row of the wave sees: a key tile outside [w_lo, w_hi) needs masking
  // (as 32-bit key numbers: key bounds lie in [0, Sk])
  int w_lo, w_hi;
  {
    int64_t l0, h0, l1, h1;
    key_range(a, klen, qlen, qw, l0, h0);
    key_range(a, klen, qlen, qw + 31, l1, h1);
    w_lo = (int)min<int64_t>(l1, a.Sk);
    // rows in [qlen, Sq) see nothing (rows past Sq are never stored)
    w_hi = (qlen < a.Sq && qw + 32 > qlen) ? w_lo : (int)min<int64_t>(h0, a.Sk);
  }

  // stage K and V rows [key0, key0 + Q_BN) straight into LDS (keys past the end arrive as
  // zeros, masked out on the tail tile)
  auto stage_tile = [&](int kt, int buf) {
    const int key0 = kt * Q_BN;
    TL::template stage_rows<Q_BN, NT>(k_lds + buf * Q_BN * D, K + (int64_t)key0 * args.sk.s, args.sk.s, a.Sk - key0);
    TL::template stage_rows<Q_BN, NT>(v_lds + buf * Q_BN * D, V + (int64_t)key0 * args.sv.s, args.sv.s, a.Sk - key0);
  };
  // a stored fp16 / q8_0 window: each tile's loads issued one tile ahead into registers,
  // converted to bf16 into LDS after the current tile's products
  constexpr int KVE = KVF == kKvQ8 ? 1 : 2;
  const char* Kst = static_cast<const char*>(args.k) + (b * args.sk.b + hk * args.sk.h) * KVE;
  const char* Vst = static_cast<const char*>(args.v) + (b * args.sv.b + hk * args.sv.h) * KVE;
  const _Float16* Ksc = a.kscale ? a.kscale + b * a.sks.b + hk * a.sks.h : nullptr;
  const _Float16* Vsc = a.vscale ? a.vscale + b * a.svs.b + hk * a.svs.h : nullptr;
  CvtStage<D, Q_BN, NT, KVF == 0 ? 1 : KVF> kcs, vcs;
  auto load_tile = [&](int kt) {
    const int64_t key0 = (int64_t)kt * Q_BN;
    kcs.load(Kst + key0 * args.sk.s * KVE, args.sk.s, Ksc ? Ksc + key0 * a.sks.s : nullptr, a.sks.s,
             a.Sk - (int)key0);
    vcs.load(Vst + key0 * args.sv.s * KVE, args.sv.s, Vsc ? Vsc + key0 * a.svs.s : nullptr, a.svs.s,
             a.Sk - (int)key0);
  };
  auto commit_tile = [&](int buf) {
    kcs.commit(k_lds + buf * Q_BN * D);
    vcs.commit(v_lds + buf * Q_BN * D);
  };

  const int G16 = lane >> 4, L16 = lane & 15;
  const int tr_row = L16 >> 2, tr_col = 16 * (G16 & 1) + 4 * (L16 & 3);

  // mask tile map: skip key tiles dead for both 64-row blocks of this workgroup
  const int nrt = (a.Sq + kMaskTile - 1) / kMaskTile;
  // candidate j: key tile kt_begin + split + j nsplit
  auto live = [&](int j) -> bool {
    const int k = kt_begin + split + j * nsplit;
    for (int rt = q0 / kMaskTile; rt <= (q0 + Q_BM - 1) / kMaskTile && rt < nrt; ++rt)
      if (tile_class(a, b, rt, k) != kTileDead) return true;  // Q_BN = kMaskTile: key tile = block
    return false;
  };
  __shared__ uint64_t live_lds[kBwdWaves];
  LiveWords lw{live_lds, -NT, {0, 0, 0, 0}};
  const int nwalk = kt_end - kt_begin;
  const int ncand = nwalk > split ? (nwalk - split + nsplit - 1) / nsplit : 0;
  auto next_live = [&](int j) {  // candidate j -> the first live one from j (ncand: none)
    if (j >= ncand) return ncand;
    return MASK && a.tiles ? lw.next(j, ncand, tid, live) : j;
  };
  auto tile_of = [&](int j) { return j < ncand ? kt_begin + split + j * nsplit : kt_end; };
  const int rt_w = qw / kMaskTile;

  // per-tile mask state of this wave, taken one tile ahead: the block class, from the
  // wave's run of classes along its row (reloaded every 64 key blocks), and, for a 0 / -inf
  // block only, this lane's row visibility word
  ClassRun run{kTileDead, -64};
  auto load_run = [&](int k) {
    run.load(a, k & ~63, rt_w < nrt ? nkt : 0, [&](int pos) { return tile_index(a, b, rt_w, pos); });
  };
  auto mask_state = [&](int k, int& cls, uint64_t& w) {
    cls = kTileBias;
    w = ~0ull;
    if (MASK && a.tiles) {
      if (k >= run.base + 64) load_run(k);  // (a longer walk: the next 64 key blocks)
      cls = run.at(k);
      if (cls == kTileBits) w = a.rowbits[(int64_t)tile_index(a, b, rt_w, k) * kMaskTile + (row - rt_w * kMaskTile)];
    }
  };

  int kj = next_live(0);
  int kt = tile_of(kj);
  int cls_cur = kTileBias;
  uint64_t wb_cur = ~0ull;
  if (kt < kt_end) {
    if constexpr (KVF == kKvBf16) {
      stage_tile(kt, 0);
    } else {
      load_tile(kt);
      commit_tile(0);
    }
    if (MASK && a.tiles) {
      load_run(kt);
      wait_vm();  // the run's classes, with the first tile
    }
    mask_state(kt, cls_cur, wb_cur);
  }
  wait_vm();
  __syncthreads();
  for (int it = 0; kt < kt_end; ++it) {
    const int buf = it & 1;
    const int kjn = next_live(kj + 1);
    const int ktn = tile_of(kjn);
    int cls_next = kTileBias;
    uint64_t wb_next = ~0ull;
    if (ktn < kt_end) {
      mask_state(ktn, cls_next, wb_next);
      if constexpr (KVF == kKvBf16)
        stage_tile(ktn, buf ^ 1);  // lands while this tile is being processed
      else
        load_tile(ktn);
    }
    const int cls = cls_cur;
    const bool bias = MASK && (cls == kTileBias || a.alibi);  // add mask values and / or ALiBi
    const bool bits = MASK && cls == kTileBits;  // 0 / -inf block: use its visibility bits
    const bf16* kb_lds = k_lds + buf * Q_BN * D;
    const bf16* vb_lds = v_lds + buf * Q_BN * D;
    const int key0 = kt * Q_BN;
    const bool edge = !(key0 >= w_lo && key0 + Q_BN <= w_hi);
    // Keys of the tile this lane's row can see, as a bit word (bit j: key key0 + j):
    // the structure (sequence ends, lengths, causal diagonal, window) and the block's
    // visibility bits (none for a dead block, computed to exact zeros like in the dK/dV
    // walk). Blocks with none of these (wave-uniform `masked` false) skip the masking.
    const bool dead = MASK && cls == kTileDead;
    const bool masked = edge || bits || dead;
    uint64_t vis = dead ? 0ull : ~0ull;
    if (masked && !dead) {
      int64_t lo, hi;
      key_range(a, klen, qlen, row, lo, hi);
      lo -= key0;
      hi -= key0;
      vis = bit_range64((int)(lo < 0 ? 0 : (lo > Q_BN ? Q_BN : lo)), (int)(hi < 0 ? 0 : (hi > Q_BN ? Q_BN : hi)));
      if (bits) vis &= wb_cur;
    }

    // one 32-key block at a time keeps the live accumulators small
    #pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T, dP^T = V dO^T: all K / V row chunks of the block requested up front
      // (in halves when two workgroups share the compute unit: the other one's work
      // covers the wait, and the operands of a half fit beside it)
      constexpr int NH = LOWREG ? 4 : 1, PH = DS / NH;
      f32x16 st = zeros16(), dpt = zeros16();
      #pragma unroll
      for (int half = 0; half < NH; ++half) {
        bf16x8 ka[PH], va[PH];
        #pragma unroll
        for (int s = 0; s < PH; ++s) {
          ka[s] = TL::read_chunk(kb_lds, 32 * kb + r32, 2 * (PH * half + s) + g);
          va[s] = TL::read_chunk(vb_lds, 32 * kb + r32, 2 * (PH * half + s) + g);
        }
        __builtin_amdgcn_sched_barrier(0);
        #pragma unroll
        for (int s = 0; s < PH; ++s) {
          mma(st, ka[s], qf[PH * half + s]);
          mma(dpt, va[s], df[PH * half + s]);
        }
      }
      // K operands of dQ += dS K (transpose reads), landing during the softmax: registers
      // 8 hh .. of this key block hold keys 32 kb + 16 hh + 8 t + 4 g + e
      bf16x8 kbt[2][DB];
      auto read_kbt = [&](int hh) {
        const int rbase = 32 * kb + 16 * hh + 4 * g + tr_row;
        #pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x4 lo = TL::read_tr(kb_lds, rbase, 32 * db + tr_col);
          const bf16x4 hi = TL::read_tr(kb_lds, rbase + 8, 32 * db + tr_col);
          kbt[hh][db] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      };
      if constexpr (!LOWREG) {
        read_kbt(0);
        read_kbt(1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // lane (query row, half g), register r -> key 32 kb + 8 (r/4) + 4 g + r%4
      if constexpr (CAP) {
        // the capped score (the mask and ALiBi add to it below) and dP - Delta times the cap's
        // derivative 1 - tanh^2
        #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float t = 1.f - 2.f * __builtin_amdgcn_rcpf(fast_exp2(st[r] * cap_k) + 1.f);
          st[r] = cap_raw * t;
          dpt[r] = (dpt[r] - dlt) * (1.f - t * t);
        }
      }
      if (BIAS && bias && a.alibi) {  // ALiBi, as in the forward (lane = row, register = key)
        const float sl = a.alibi[h] * args.inv_scale;
        const float base = (float)((int64_t)key0 + 32 * kb + 4 * g - a.q_offset - row);
        #pragma unroll
        for (int r = 0; r < 16; ++r) st[r] -= sl * fabsf(base + (float)(8 * (r >> 2) + (r & 3)));
      }
      if (BIAS && bias && a.mask) {  // additive mask values, 4 keys at a time (keys past the end read 0)
        const float* mr = a.mask + b * a.mask_sb + h * a.mask_sh + (int64_t)min(row, a.Sq - 1) * a.mask_sq;
        #pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int k4 = key0 + 32 * kb + 8 * rr + 4 * g;
          float mv[4];
          if (k4 + 3 < a.Sk && args.mask_vec4) {
            const f32x4 m4 = *reinterpret_cast<const f32x4*>(mr + k4);
            mv[0] = m4[0]; mv[1] = m4[1]; mv[2] = m4[2]; mv[3] = m4[3];
          } else {
            #pragma unroll
            for (int e = 0; e < 4; ++e) mv[e] = (k4 + e < a.Sk) ? mr[k4 + e] : 0.f;
          }
          #pragma unroll
          for (int e = 0; e < 4; ++e) st[4 * rr + e] += mv[e] * args.inv_scale;
        }
      }
      if (masked) {  // hidden scores -> -inf (P = 0); bit 8 rr + e of w <-> register 4 rr + e
        const uint32_t w = (uint32_t)(vis >> (32 * kb + 4 * g));
        #pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = ninf_unless_bit(st[r], w, 8 * (r >> 2) + (r & 3));
      }
      #pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = fast_exp2(fmaf(st[r], cs, -lse2));
      #pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = st[r] * (CAP ? dpt[r] : dpt[r] - dlt);
      if constexpr (MG) add_mask_grad(args, b, h, row, key0 + 32 * kb + 4 * g, st);
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if constexpr (LOWREG) read_kbt(hh);  // (two workgroups per unit: read when needed)
        bf16x8 dsf;
        pack8(dsf, st, 8 * hh);
        #pragma unroll
        for (int db = 0; db < DB; ++db) mma_acc(dq[db], dsf, kbt[hh][db]);
      }
    }
    if constexpr (KVF != kKvBf16) {
      if (ktn < kt_end) commit_tile(buf ^ 1);
    }
    wait_vm();
    __syncthreads();
    kt = ktn;
    kj = kjn;
    cls_cur = cls_next;
    wb_cur = wb_next;
  }

  settle_acc(dq);
  // split walks store this split's fp32 slice (unscaled), summed by a reduce pass; the
  // tile buffers stage the results once every wave has left the walk
  const int rows = max(0, min(32, a.Sq - qw));
  const RowSink sq =
      nsplit > 1
          ? RowSink{reinterpret_cast<char*>(plan.dq_part + (int64_t)split * a.B * a.Hq * a.Sq * D +
                                            (((int64_t)b * a.Hq + h) * a.Sq + qw) * D),
                    (int64_t)D * 4, rows, 1}
          : RowSink{reinterpret_cast<char*>(static_cast<bf16*>(plan.dq) + b * plan.sdq.b + h * plan.sdq.h +
                                            (int64_t)qw * plan.sdq.s),
                    plan.sdq.s * 2, rows, 0};
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * D;
  __syncthreads();
  store_block<D>(dq, nsplit > 1 ? 1.f : a.scale, stage, lane, sq);
}

// ---------------------------------------------------------------------------
// dQ workgroup over stored dS
// ---------------------------------------------------------------------------
// dQ = scale dS K from the dS blocks the dK/dV walk stored (dS = P (dP - Delta) is the same
// quantity the dQ walk recomputes from S and dP, already rounded to bf16 the way both walks
// feed it to their products). What is left per key tile is one product reading dS once from
// memory, so the pass streams dS: a workgroup owns 256 query rows (each wave one 64-row tile,
// the rows of one dS block) and keeps two 64-key tiles in flight through a ring of three
// stages in LDS, each a K tile (read by all four waves) and, per wave, the half block of
// its row tile holding the tile's keys (read by that wave only). The dS operand of a 16-key
// product is two transpose reads of the stored chunks (each 16-lane group reads 128
// contiguous bytes). A wave uses a block only if the dK/dV walk visited it (the same row
// range and mask block test): a block it skipped holds no data, and its scores are all
// hidden, so the wave's products for it are skipped.
template <int D, bool MASK>
__device__ __forceinline__ void dqds_unit(const BwdArgs& args, const BwdPlan& plan, int unit, char* smem) {
  constexpr int DB = D / 32;
  constexpr int SB = kDsBlock / 2;            // half a dS block: 64 rows x 64 keys
  constexpr int QM = kDsRows;                 // query rows per workgroup
  constexpr int KT = Q_BN * D * 2;            // bytes of a staged K tile
  constexpr int STAGE = KT + kBwdWaves * SB;  // one ring stage
  constexpr int NS = 3;                       // ring stages: two tiles in flight
  // VMEM instructions per thread and stage (K tile rows, then the wave's 8 KB of dS): the
  // wait for a stage lets the next stage's loads stay outstanding
  constexpr int KLOADS = Q_BN * (D / 8) / NT, SLOADS = SB / 1024;
  static_assert(QM == 64 * kBwdWaves, "one 64-row dS tile per wave");
  using TL = Tile<D>;

  const AttnShape& a = args.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) from here on
  const int g = lane >> 5;
  const QUnit u = q_unit_of(a, plan, unit);
  const int qt = u.qt, b = u.b, h = u.h, split = u.split, nsplit = u.nsplit;
  const int hk = h / a.G;
  const int q0 = qt * QM;
  const int qw = q0 + KV_BM * wave;  // the wave's 64 rows: dS row tile rt_w
  const int rt_w = qw / KV_BM;
  const bf16* K = static_cast<const bf16*>(args.k) + b * args.sk.b + hk * args.sk.h;
  const char* dsw = plan.ds + (((int64_t)b * a.Hq + h) * plan.ds_nku * plan.ds_nrt + rt_w) * kDsBlock;
  const uint32_t ds_bytes = rt_w < plan.ds_nrt ? (uint32_t)SB : 0u;  // (no row tile: zeros, never used)

  // (accumulators in arch VGPRs: the products sit under a wave-uniform branch, across which
  // accumulators in AGPRs would be copied out and back every tile)
  f32x16 dq[2][DB];
  #pragma unroll
  for (int qb = 0; qb < 2; ++qb)
    #pragma unroll
    for (int db = 0; db < DB; ++db) dq[qb][db] = zeros16();

  // the key tiles the workgroup's rows can see by the structure (as in the dQ walk)
  const int klen = klen_of(a, b), qlen = qlen_of(a, b);
  const int nkt = (a.Sk + Q_BN - 1) / Q_BN;
  int kt_begin = 0, kt_end = 0;
  if (q0 < qlen) {
    int64_t lo, hi, lo1, hi1;
    key_range(a, klen, qlen, q0, lo, hi);
    key_range(a, klen, qlen, min(q0 + QM, qlen) - 1, lo1, hi1);
    kt_begin = (int)min<int64_t>(lo / Q_BN, nkt);
    kt_end = hi1 > lo ? (int)min<int64_t>((hi1 + Q_BN - 1) / Q_BN, nkt) : kt_begin;
    if (kt_end < kt_begin) kt_end = kt_begin;
  }

  // stage key tile kt into ring slot `slot`: its K rows (keys past the end arrive as zeros)
  // and this wave's half of dS block (rt_w, kt / 2), the latter with the non-temporal hint
  // (read once: LM step 2.7% faster than with cached loads)
  auto stage_tile = [&](int kt, int slot) {
    char* base = smem + slot * STAGE;
    const int key0 = kt * Q_BN;
    TL::template stage_rows<Q_BN, NT>(TL::lds_addr(base), K + (int64_t)key0 * args.sk.s, args.sk.s, a.Sk - key0);
    const u32x4 rsrc = raw_rsrc(dsw + (int64_t)(kt >> 1) * plan.ds_nrt * kDsBlock + (kt & 1) * SB, ds_bytes);
    const uint32_t dst = TL::lds_addr(base + KT + wave * SB);
    #pragma unroll
    for (int i = 0; i < SLOADS; ++i) TL::dma16nt(rsrc, (uint32_t)(1024 * i + 16 * lane), 0u, dst + 1024u * i);
  };

  // did the dK/dV walk store block (rt_w, ku)?
  const int nct = (a.Sk + kMaskTile - 1) / kMaskTile;
  auto visited = [&](int ku) -> bool {
    int t0, t1;
    kv_row_tiles(a, klen, qlen, ku * KV_BN, t0, t1);
    if (rt_w < t0 || rt_w >= t1) return false;
    if (MASK && a.tiles) {
      for (int ct = ku * (KV_BN / kMaskTile); ct < (ku + 1) * (KV_BN / kMaskTile) && ct < nct; ++ct)
        if (tile_class(a, b, rt_w, ct) != kTileDead) return true;
      return false;
    }
    return true;
  };

  // mask tile map: skip key tiles dead for every 64-row block of this workgroup
  const int nrt = (a.Sq + kMaskTile - 1) / kMaskTile;
  auto live = [&](int j) -> bool {  // candidate j: key tile kt_begin + split + j nsplit
    const int k = kt_begin + split + j * nsplit;
    for (int rt = q0 / kMaskTile; rt <= (q0 + QM - 1) / kMaskTile && rt < nrt; ++rt)
      if (tile_class(a, b, rt, k) != kTileDead) return true;
    return false;
  };
  __shared__ uint64_t live_lds[kBwdWaves];
  LiveWords lw{live_lds, -NT, {0, 0, 0, 0}};
  const int nwalk = kt_end - kt_begin;
  const int ncand = nwalk > split ? (nwalk - split + nsplit - 1) / nsplit : 0;
  auto next_live = [&](int j) {
    if (j >= ncand) return ncand;
    return MASK && a.tiles ? lw.next(j, ncand, tid, live) : j;
  };
  auto tile_of = [&](int j) { return j < ncand ? kt_begin + split + j * nsplit : kt_end; };

  // the dS operand: lane L of 16-lane group G reads keys 4 g + L / 4 (+ 8) of a 16-key step,
  // rows 16 (G & 1) + 4 (L & 3) .. + 3 of a 32-row block; in the stored order that is chunk
  // (qb, G & 1, key, L & 1), byte 8 ((L >> 1) & 1)
  const int G16 = lane >> 4, L16 = lane & 15, hs = G16 & 1;
  const uint32_t a_off =
      (uint32_t)(((hs * 32 + ((4 * g + (L16 >> 2)) ^ (4 * hs))) * 2 + (L16 & 1)) * 16 + ((L16 >> 1) & 1) * 8);
  const int tr_row = L16 >> 2, tr_col = 16 * (G16 & 1) + 4 * (L16 & 3);
  auto read_tr_at = [](const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(__attribute__((address_space(3))) char*)p);
  };

  int kj = next_live(0);
  int kt = tile_of(kj);
  int kjn = next_live(kj + 1);
  int ktn = tile_of(kjn);
  if (kt < kt_end) stage_tile(kt, 0);
  if (ktn < kt_end) {
    stage_tile(ktn, 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_enc(KLOADS + SLOADS));  // the first stage
  } else {
    wait_vm();
  }
  __syncthreads();
  int ku_c = -1;
  bool ok = false;
  for (int slot = 0, slot_n = 1, slot_f = 2; kt < kt_end;) {
    const int kjf = next_live(kjn + 1);
    const int ktf = tile_of(kjf);
    if (ktf < kt_end) stage_tile(ktf, slot_f);  // two tiles ahead (its slot was read last tile)
    if ((kt >> 1) != ku_c) {
      ku_c = kt >> 1;
      ok = visited(ku_c);
    }
    if (ok) {
      const bf16* kb_lds = reinterpret_cast<const bf16*>(smem + slot * STAGE);
      const char* sa = smem + slot * STAGE + KT + wave * SB + a_off;
      #pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          // K operands (transpose reads): keys 32 kb + 16 hh + 4 g + e and + 8
          const int rbase = 32 * kb + 16 * hh + 4 * g + tr_row;
          bf16x8 kbt[DB];
          #pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x4 lo = TL::read_tr(kb_lds, rbase, 32 * db + tr_col);
            const bf16x4 hi = TL::read_tr(kb_lds, rbase + 8, 32 * db + tr_col);
            kbt[db] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          #pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const char* p = sa + 2048 * qb + 4096 * kb + 512 * hh;
            const bf16x4 lo = read_tr_at(p), hi = read_tr_at(p + 256);
            const bf16x8 dsf = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            #pragma unroll
            for (int db = 0; db < DB; ++db) mma(dq[qb][db], dsf, kbt[db]);
          }
        }
      }
    }
    if (ktf < kt_end)
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(KLOADS + SLOADS));  // the next stage (not the one after)
    else
      wait_vm();
    __syncthreads();
    kt = ktn;
    kj = kjn;
    ktn = ktf;
    kjn = kjf;
    const int s0 = slot;
    slot = slot_n;
    slot_n = slot_f;
    slot_f = s0;
  }

  // split walks store this split's fp32 slice (unscaled), summed by a reduce pass; the ring
  // stages the results once every wave has left the walk
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * D;
  #pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r0 = qw + 32 * qb;
    const int rows = max(0, min(32, a.Sq - r0));
    const RowSink sq =
        nsplit > 1
            ? RowSink{reinterpret_cast<char*>(plan.dq_part + (int64_t)split * a.B * a.Hq * a.Sq * D +
                                              (((int64_t)b * a.Hq + h) * a.Sq + r0) * D),
                      (int64_t)D * 4, rows, 1}
            : RowSink{reinterpret_cast<char*>(static_cast<bf16*>(plan.dq) + b * plan.sdq.b + h * plan.sdq.h +
                                              (int64_t)r0 * plan.sdq.s),
                      plan.sdq.s * 2, rows, 0};
    store_block<D>(dq[qb], nsplit > 1 ? 1.f : a.scale, stage, lane, sq);
  }
}

// Units whose mask blocks carry additive values run a body compiled with the
// mask-value reads; all others (dead / open / 0-or--inf blocks) a body without them,
// which keeps that code and its registers out of the common loop.
template <int D, bool CAUSAL, bool MASK, bool CAP = false, int KVF = 0, bool MG = false, bool ST = false>
__global__ __launch_bounds__(NT) void bwd_bf16_kernel(const BwdArgs args, const BwdPlan plan) {
  constexpr int KV_LDS = 3 * 2 * KV_BM * D * 2 + 2 * 3 * KV_BM * 16 * 2;
  constexpr int Q_LDS = 2 * 2 * Q_BN * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[KV_LDS > Q_LDS ? KV_LDS : Q_LDS];
  const int blk = blockIdx.x;
  const AttnShape& a = args.a;
  if (blk < plan.n_kv_units) {
    const KvUnit u = kv_unit_of(a, plan, blk);
    const int nrb = (a.Sq + kMaskTile - 1) / kMaskTile, cb0 = u.kt * (KV_BN / kMaskTile);
    // whole pairs by the structure: no causal diagonal or window, every key below the length
    const bool whole = !CAUSAL && !CAP && a.wl < 0 && a.wr < 0 && (u.kt + 1) * KV_BN <= klen_of(a, u.b);
    if (MASK && any_bias_block(a, u.b, 0, nrb, cb0, KV_BN / kMaskTile)) {
      dkdv_unit<D, CAUSAL, MASK, true, CAP, KVF, ST>(args, plan, blk, smem);
    } else if (MASK && all_open_blocks(a, u.b, 0, nrb, cb0, KV_BN / kMaskTile)) {
      if (whole)
        dkdv_unit<D, CAUSAL, false, false, CAP, KVF, ST, !CAUSAL && !CAP>(args, plan, blk, smem);
      else
        dkdv_unit<D, CAUSAL, false, false, CAP, KVF, ST>(args, plan, blk, smem);
    } else if (!MASK && whole) {
      dkdv_unit<D, CAUSAL, false, false, CAP, KVF, ST, !CAUSAL && !CAP>(args, plan, blk, smem);
    } else {
      dkdv_unit<D, CAUSAL, MASK, false, CAP, KVF, ST>(args, plan, blk, smem);
    }
  } else if constexpr (!ST) {
    const int unit = blk - plan.n_kv_units;
    const QUnit u = q_unit_of(a, plan, unit);
    if (MASK && any_bias_block(a, u.b, u.qt * (Q_BM / kMaskTile), Q_BM / kMaskTile, 0,
                               (a.Sk + kMaskTile - 1) / kMaskTile))
      dq_unit<D, CAUSAL, MASK, true, false, CAP, KVF, MG>(args, plan, unit, smem);
    else
      dq_unit<D, CAUSAL, MASK, false, false, CAP, KVF, MG>(args, plan, unit, smem);
  }
}

// The role-split dK/dV walk as a kernel of its own, two workgroups per compute unit; the
// dQ walk follows as bwd_dq_kernel. (One launch for both would need the two walks'
// registers together, beyond the 256 a wave gets at two workgroups per unit.)
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(NT, 2) void bwd_role_kernel(const BwdArgs args, const BwdPlan plan) {
  constexpr int KV_LDS = (4 * KV_BM * D + 2 * 2 * KV_BM * 8 + 2 * 2 * 64 * 16) * 2;
  __shared__ __attribute__((aligned(16))) char smem[KV_LDS];
  const int blk = blockIdx.x;
  const AttnShape& a = args.a;
  const KvUnit u = kv_unit_of(a, plan, blk);
  if (MASK && any_bias_block(a, u.b, 0, (a.Sq + kMaskTile - 1) / kMaskTile, u.kt * (kBwdRoleKeys / kMaskTile),
                             kBwdRoleKeys / kMaskTile))
    dkdv_role_unit<D, CAUSAL, MASK, true>(args, plan, blk, smem);
  else
    dkdv_role_unit<D, CAUSAL, MASK, false>(args, plan, blk, smem);
}

// The dQ walk as a kernel of its own: its registers fit two workgroups per compute unit
// (the dK/dV walk's do not), so that one workgroup's LDS and memory waits are covered by
// the other's products. Launched after the dK/dV-only grid when the plan asks for it.
template <int D, bool CAUSAL, bool MASK, bool CAP = false, int KVF = 0, bool MG = false>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(const BwdArgs args, const BwdPlan plan) {
  constexpr int Q_LDS = 2 * 2 * Q_BN * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[Q_LDS];
  const int unit = blockIdx.x;
  const AttnShape& a = args.a;
  const QUnit u = q_unit_of(a, plan, unit);
  if (MASK && any_bias_block(a, u.b, u.qt * (Q_BM / kMaskTile), Q_BM / kMaskTile, 0,
                             (a.Sk + kMaskTile - 1) / kMaskTile))
    dq_unit<D, CAUSAL, MASK, true, true, CAP, KVF, MG>(args, plan, unit, smem);
  else
    dq_unit<D, CAUSAL, MASK, false, true, CAP, KVF, MG>(args, plan, unit, smem);
}

// dQ over the dS blocks the dK/dV-only grid stored before it (one workgroup per compute
// unit, its loads two tiles ahead)
template <int D, bool MASK>
__global__ __launch_bounds__(NT, 1) void bwd_dqds_kernel(const BwdArgs args, const BwdPlan plan) {
  __shared__ __attribute__((aligned(16))) char smem[3 * (Q_BN * D * 2 + kBwdWaves * kDsBlock / 2)];
  dqds_unit<D, MASK>(args, plan, blockIdx.x, smem);
}

template <int D, bool CAUSAL, bool MASK, bool CAP = false, int KVF = 0, bool MG = false>
hipError_t launch_cm(const BwdArgs& args, const BwdPlan& plan, hipStream_t stream) {
  // (a separate dQ kernel may go to a second stream, joined by the caller)
  hipStream_t dq_stream = plan.dq_stream ? plan.dq_stream : stream;
  if constexpr (KVF == 0 && !MG) {
    if (plan.ds) {  // the dK/dV walk stores dS, then the dQ pass over it
      if (plan.n_kv_units > 0)
        hipLaunchKernelGGL((bwd_bf16_kernel<D, CAUSAL, MASK, CAP, 0, false, true>), dim3(plan.n_kv_units), dim3(NT), 0,
                           stream, args, plan);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || plan.n_q_units == 0) return e;
      hipLaunchKernelGGL((bwd_dqds_kernel<D, MASK>), dim3(plan.n_q_units), dim3(NT), 0, stream, args, plan);
      return hipGetLastError();
    }
  }
  if constexpr (!CAP && KVF == 0) {
    if (plan.kv_role) {
      if (plan.n_kv_units > 0)
        hipLaunchKernelGGL((bwd_role_kernel<D, CAUSAL, MASK>), dim3(plan.n_kv_units), dim3(NT), 0, stream, args, plan);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || plan.n_q_units == 0) return e;
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, MASK, CAP, KVF, MG>), dim3(plan.n_q_units), dim3(NT), 0, dq_stream, args,
                         plan);
      return hipGetLastError();
    }
  }
  if (!plan.dq_separate) {
    hipLaunchKernelGGL((bwd_bf16_kernel<D, CAUSAL, MASK, CAP, KVF, MG>), dim3(plan.n_kv_units + plan.n_q_units), dim3(NT), 0,
                       stream, args, plan);
    return hipGetLastError();
  }
  if (plan.n_kv_units > 0)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, CAUSAL, MASK, CAP, KVF, MG>), dim3(plan.n_kv_units), dim3(NT), 0, stream, args,
                       plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.n_q_units == 0) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, MASK, CAP, KVF, MG>), dim3(plan.n_q_units), dim3(NT), 0, dq_stream, args, plan);
  return hipGetLastError();
}

template <int D>
hipError_t launch_t(const BwdArgs& args, const BwdPlan& plan, hipStream_t stream) {
  const bool causal = args.a.causal != 0, mask = args.a.mask != nullptr || args.a.alibi != nullptr;
  if (args.a.kvf == kKvQ8)  // a stored window: no dense mask, ALiBi or softcap (checked on the host)
    return causal ? launch_cm<D, true, false, false, kKvQ8>(args, plan, stream)
                  : launch_cm<D, false, false, false, kKvQ8>(args, plan, stream);
  if (args.a.kvf == kKvF16)
    return causal ? launch_cm<D, true, false, false, kKvF16>(args, plan, stream)
                  : launch_cm<D, false, false, false, kKvF16>(args, plan, stream);
  if (args.a.softcap > 0.f) {  // the capped walks (with a dense mask or ALiBi, added after the cap)
    if (mask) return causal ? launch_cm<D, true, true, true>(args, plan, stream) : launch_cm<D, false, true, true>(args, plan, stream);
    return causal ? launch_cm<D, true, false, true>(args, plan, stream) : launch_cm<D, false, false, true>(args, plan, stream);
  }
  if (args.dbias)  // (a dense mask, no softcap: checked on the host)
    return causal ? launch_cm<D, true, true, false, 0, true>(args, plan, stream)
                  : launch_cm<D, false, true, false, 0, true>(args, plan, stream);
  if (causal && mask) return launch_cm<D, true, true>(args, plan, stream);
  if (causal) return launch_cm<D, true, false>(args, plan, stream);
  if (mask) return launch_cm<D, false, true>(args, plan, stream);
  return launch_cm<D, false, false>(args, plan, stream);
}

}  // namespace

void plan_bwd_bf16(const AttnShape& a, int kv_split, int q_split, int q_tiles_split, int dq_separate,
                   BwdPlan* plan, int kv_role, int dq_ds) {
  plan->dq_separate = dq_separate;
  plan->kv_role = kv_role;
  plan->ds = nullptr;  // (set by the caller for the dQ pass over stored dS)
  plan->dq_stream = nullptr;  // (set by the caller to run the dQ kernel beside the dK/dV kernel)
  plan->ds_nrt = (a.Sq + KV_BM - 1) / KV_BM;
  plan->ds_nku = (a.Sk + KV_BN - 1) / KV_BN;
  const int kvb = kv_role ? kBwdRoleKeys : KV_BN;
  const int nkt = (a.Sk + kvb - 1) / kvb;
  plan->q_bm = dq_ds ? kDsRows : Q_BM;
  const int nqt = (a.Sq + plan->q_bm - 1) / plan->q_bm;
  if (dq_ds) q_tiles_split = min((q_tiles_split * Q_BM + kDsRows - 1) / kDsRows, nqt);
  plan->kv_split = kv_split;
  plan->q_split = q_split;
  plan->n_kv_units = nkt * a.B * a.Hkv * kv_split;
  plan->q_tiles_split = q_split > 1 ? q_tiles_split : 0;
  plan->n_q_units = (nqt - plan->q_tiles_split + plan->q_tiles_split * q_split) * a.B * a.Hq;
}

hipError_t launch_bwd_bf16(const BwdArgs& args, const BwdPlan& plan, hipStream_t stream) {
  return args.a.D == 64 ? launch_t<64>(args, plan, stream) : launch_t<128>(args, plan, stream);
}

}  // namespace fa
