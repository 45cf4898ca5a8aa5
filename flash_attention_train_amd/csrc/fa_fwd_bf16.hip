// fa_fwd_bf16.hip -- the bf16 forward: O and the per-row LSE.
//
// Same mathematics as the generic forward (online softmax over key tiles, the
// LSE kept for the backward -- "Flash Attn Training" skill page, section 6,
// trap 3), organised for gfx950's matrix cores and LDS:
//
//  * one workgroup of 4 waves per (batch, head, 32*4*QB-row query tile); each
//    wave owns QB blocks of 32 query rows, held in registers as the B operand
//    of S^T = K Q^T for the whole walk;
//  * K and V tiles of BN keys are copied row-major into LDS by direct global-to-LDS
//    loads (no registers), double-buffered: the next tile's loads are issued into the
//    other buffer before the current tile's products, so one barrier per tile suffices;
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
#include "fa_tile.h"

namespace fa {

namespace {

__device__ __forceinline__ f32x16 zeros16() {
  f32x16 z;
  #pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// KS = 2 splits the keys of a query tile over two halves of the workgroup (for problems
// with too few query tiles to fill the GPU): waves 0-1 and 2-3 own the same 64 rows, take
// alternate live key tiles, and merge their (max, sum, O) in LDS at the end.
// SPLIT: workgroup blockIdx.z walks only the blockIdx.z-th contiguous share of the live
// range's key tiles and leaves its unnormalised rows to the merge pass.
// KVF: K and V stored as bf16 (0), fp16 (1) or q8_0 (2); the last two are converted to bf16
// on their way into LDS (their tiles' loads issued one tile ahead into registers, converted
// and written after the current tile's products), so a quantised window is read in place.
template <int D, int QB, int BN, bool CAUSAL, bool MASK, int KS, bool SPLIT = false, int KVF = 0>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1) void fwd_bf16_kernel(const FwdArgs args) {
  static_assert(KVF == 0 || (KS == 1 && QB == 1 && BN == 64), "stored K / V formats take the default walk");
  constexpr int NW = 4;
  constexpr int RB = NW / KS;       // waves (row blocks) per key half
  constexpr int BM = RB * QB * 32;  // query rows per workgroup
  constexpr int KB = BN / 32;       // 32-key blocks per tile
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int NTS = 64 * RB;      // threads staging one key half's tiles
  using TL = Tile<D>;
  __shared__ __attribute__((aligned(16))) bf16 kv_lds[2][KS][2][BN * D];  // K and V: [key half][buffer]
  bf16(&k_lds)[KS][2][BN * D] = kv_lds[0];
  bf16(&v_lds)[KS][2][BN * D] = kv_lds[1];

  const AttnShape& a = args.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) from here on
  const int rb = wave % RB, kh = wave / RB;                    // row block, key half
  const uint32_t k_lds32 = TL::lds_addr(k_lds[kh][0]), v_lds32 = TL::lds_addr(v_lds[kh][0]);  // (staging destinations)
  const int g = lane >> 5, r32 = lane & 31;
  // Workgroups are dispatched in linear order with x fastest: x walks (batch, head) and y
  // the query tiles from the last, so every head's longest causal walks go out first.
  const int h = blockIdx.x % a.Hq, b = blockIdx.x / a.Hq;
  const int qt = gridDim.y - 1 - blockIdx.y;
  const int q0 = qt * BM;
  const int qw = q0 + rb * QB * 32;            // first row of this wave
  const int hk = h / a.G;
  const float cs = a.scale * kLog2e;           // scale > 0 (checked on the host)
  // logit softcap c in raw score units: S -> (c / scale) tanh(S scale / c), with
  // tanh(x) = 1 - 2 / (e^(2x) + 1) from the hardware exp2 and reciprocal (absolute error a
  // few ulp of 1; e^(2x) overflowing to inf gives 1, underflowing to 0 gives -1)
  const bool capped = a.softcap > 0.f;
  const float cap_k = capped ? 2.f * kLog2e * a.scale / a.softcap : 0.f;
  const float cap_raw = a.softcap * args.inv_scale;

  const bf16* Q = static_cast<const bf16*>(args.q) + b * args.sq.b + h * args.sq.h;
  const bf16* K = static_cast<const bf16*>(args.k) + b * args.sk.b + hk * args.sk.h;
  const bf16* V = static_cast<const bf16*>(args.v) + b * args.sv.b + hk * args.sv.h;

  // Q rows as B operands: lane (row r32, half g) holds d = 16 s + 8 g .. + 7
  bf16x8 qf[QB][DS];
  #pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // (rows past the end read the last row and are never stored; a zeroing branch would
    // make the loads wait here)
    const int64_t row_c = min(qw + 32 * qb + r32, a.Sq - 1);
    #pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[qb][s] = *reinterpret_cast<const bf16x8*>(Q + row_c * args.sq.s + 16 * s + 8 * g);
  }

  f32x16 oacc[QB][DB];
  float base[QB], lsum[QB];
  #pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    #pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = zeros16();
    base[qb] = neg_inf();
    lsum[qb] = 0.f;
  }

  // keys the workgroup's rows can see by the structure (sequence ends, causal diagonal,
  // key and query lengths, window): from the first row's lower end to the last visible
  // row's upper end (both ends move right with the row)
  const int klen = klen_of(a, b), qlen = qlen_of(a, b);
  const int nkt = (a.Sk + BN - 1) / BN;
  int kt_begin = 0, kt_end = 0;
  if (q0 < qlen) {
    int64_t lo, hi, lo1, hi1;
    key_range(a, klen, qlen, q0, lo, hi);
    key_range(a, klen, qlen, min(q0 + BM, qlen) - 1, lo1, hi1);
    kt_begin = (int)min<int64_t>(lo / BN, nkt);
    kt_end = hi1 > lo ? (int)min<int64_t>((hi1 + BN - 1) / BN, nkt) : 0;
    if (kt_end < kt_begin) kt_end = kt_begin;
  }
  // the wave's rows: every key tile outside [w_lo, w_hi) needs per-element masking
  // (as 32-bit key numbers: key bounds lie in [0, Sk])
  int w_lo, w_hi;
  {
    int64_t l0, h0, l1, h1;
    key_range(a, klen, qlen, qw, l0, h0);
    key_range(a, klen, qlen, qw + QB * 32 - 1, l1, h1);
    w_lo = (int)min<int64_t>(l1, a.Sk);  // the largest lower end
    // rows in [qlen, Sq) see nothing (rows past Sq are never stored)
    w_hi = (qlen < a.Sq && qw + QB * 32 > qlen) ? w_lo : (int)min<int64_t>(h0, a.Sk);
  }
  if constexpr (SPLIT) {  // this workgroup's share of [kt_begin, kt_end)
    const int per = (kt_end - kt_begin + (int)gridDim.z - 1) / (int)gridDim.z;
    kt_begin = min(kt_end, kt_begin + (int)blockIdx.z * per);
    kt_end = min(kt_end, kt_begin + per);
  }

  // tile staging: K and V rows [key0, key0 + BN) straight into LDS; keys past the end
  // arrive as zeros (masked out, P = 0, on the tail tile)
  // (with KS = 2 each key half stages its own tile with its own two waves)
  auto stage_tile = [&](int kt, int buf) {
    const int key0 = kt * BN;
    TL::template stage_rows<BN, NTS>(k_lds32 + (uint32_t)buf * (BN * D * 2), K + (int64_t)key0 * args.sk.s, args.sk.s,
                                     a.Sk - key0, rb);
    TL::template stage_rows<BN, NTS>(v_lds32 + (uint32_t)buf * (BN * D * 2), V + (int64_t)key0 * args.sv.s, args.sv.s,
                                     a.Sk - key0, rb);
  };
  // stored fp16 / q8_0 tiles: loads one tile ahead, conversion into LDS after the products
  constexpr int KVE = KVF == kKvQ8 ? 1 : 2;  // bytes per stored element
  const char* Kst = static_cast<const char*>(args.k) + (b * args.sk.b + hk * args.sk.h) * KVE;
  const char* Vst = static_cast<const char*>(args.v) + (b * args.sv.b + hk * args.sv.h) * KVE;
  const _Float16* Ksc = a.kscale ? a.kscale + b * a.sks.b + hk * a.sks.h : nullptr;
  const _Float16* Vsc = a.vscale ? a.vscale + b * a.svs.b + hk * a.svs.h : nullptr;
  CvtStage<D, BN, NTS, KVF == 0 ? 1 : KVF> kcs, vcs;
  auto load_tile = [&](int kt) {
    const int64_t key0 = (int64_t)kt * BN;
    kcs.load(Kst + key0 * args.sk.s * KVE, args.sk.s, Ksc ? Ksc + key0 * a.sks.s : nullptr, a.sks.s,
             a.Sk - (int)key0, rb);
    vcs.load(Vst + key0 * args.sv.s * KVE, args.sv.s, Vsc ? Vsc + key0 * a.svs.s : nullptr, a.svs.s,
             a.Sk - (int)key0, rb);
  };
  auto commit_tile = [&](int buf) {
    kcs.commit(k_lds[kh][buf], rb);
    vcs.commit(v_lds[kh][buf], rb);
  };

  // With a mask tile map, key tiles whose mask blocks are dead for every row block
  // of this workgroup are skipped outright (no load, no products); per wave, a dead
  // block skips the products and an open block skips the mask reads.
  const int nrt = (a.Sq + kMaskTile - 1) / kMaskTile;
  const int rt_w = qw / kMaskTile;  // the wave's QB * 32 rows lie in one 64-row block
  auto live = [&](int kt) -> bool {
    if (!MASK || !a.tiles) return true;
    const int ct = (kt * BN) / kMaskTile;
    for (int rt = q0 / kMaskTile; rt <= (q0 + BM - 1) / kMaskTile && rt < nrt; ++rt)
      if (tile_class(a, b, rt, ct) != kTileDead) return true;
    return false;
  };
  // The live key tiles of the workgroup, 256 at a time, as bit words: found by all threads
  // at once and kept in scalar registers, so that a step of the walk waits on neither a
  // class load nor an LDS read.
  __shared__ uint64_t live_lds[LiveWords::kWaves];
  LiveWords lw{live_lds, -LiveWords::kThreads, {0, 0, 0, 0}};
  auto next_live = [&](int kt) {
    if (!MASK || !a.tiles) return kt < kt_end ? kt : kt_end;
    return lw.next(kt, kt_end, tid, live);
  };

  // Per-tile mask state of this wave. The classes of its row block along the keys come as
  // a run, one per lane and 64 key blocks per load (a longer walk reloads when it gets
  // there), so a tile's class is one readlane; the row visibility words are loaded only
  // for a 0 / -inf block, one tile ahead (they complete under the end-of-iteration wait).
  const int nct = (a.Sk + kMaskTile - 1) / kMaskTile;
  ClassRun run{kTileDead, -64};
  auto load_run = [&](int ct) {
    run.load(a, ct & ~63, rt_w < nrt ? nct : 0, [&](int pos) { return tile_index(a, b, rt_w, pos); });
  };
  auto mask_state = [&](int kt, int& cls, uint64_t (&w)[QB]) {
    cls = kTileBias;
    #pragma unroll
    for (int qb = 0; qb < QB; ++qb) w[qb] = ~0ull;
    if (MASK && a.tiles) {
      const int ct = (kt * BN) / kMaskTile;
      if (ct >= run.base + 64) load_run(ct);
      cls = run.at(ct);
      if (cls == kTileBits) {
        const int64_t base = (int64_t)tile_index(a, b, rt_w, ct) * kMaskTile - rt_w * kMaskTile;
        #pragma unroll
        for (int qb = 0; qb < QB; ++qb) w[qb] = a.rowbits[base + qw + 32 * qb + r32];
      }
    }
  };

  // The walk goes in steps of KS live tiles (tk[0] < tk[1] ...); this wave's tile is tk[kh].
  // (the first run of classes lands under the wait of the first search for live tiles)
  if (MASK && a.tiles) load_run((kt_begin * BN) / kMaskTile);
  int tk[KS];
  tk[0] = next_live(kt_begin);
  #pragma unroll
  for (int j = 1; j < KS; ++j) tk[j] = tk[j - 1] < kt_end ? next_live(tk[j - 1] + 1) : kt_end;
  int kt = tk[kh];
  int cls_cur = kTileBias;
  uint64_t wb_cur[QB];
  #pragma unroll
  for (int qb = 0; qb < QB; ++qb) wb_cur[qb] = ~0ull;
  if (kt < kt_end) {
    if constexpr (KVF == 0) {
      stage_tile(kt, 0);
    } else {
      load_tile(kt);
      commit_tile(0);
    }
    mask_state(kt, cls_cur, wb_cur);
  }
  wait_vm();
  __syncthreads();

  // transpose-read addressing inside a 16-lane group
  const int G16 = lane >> 4, L16 = lane & 15;
  const int tr_row = L16 >> 2, tr_col = 16 * (G16 & 1) + 4 * (L16 & 3);

  for (int it = 0; tk[0] < kt_end; ++it) {
    const int buf = it & 1;
    int tn[KS];
    tn[0] = tk[KS - 1] < kt_end ? next_live(tk[KS - 1] + 1) : kt_end;
    #pragma unroll
    for (int j = 1; j < KS; ++j) tn[j] = tn[j - 1] < kt_end ? next_live(tn[j - 1] + 1) : kt_end;
    const int ktn = tn[kh];
    const bool more = ktn < kt_end;
    int cls_next = kTileBias;
    uint64_t wb_next[QB];
    #pragma unroll
    for (int qb = 0; qb < QB; ++qb) wb_next[qb] = ~0ull;
    if (more) {
      mask_state(ktn, cls_next, wb_next);
      if constexpr (KVF == 0)
        stage_tile(ktn, buf ^ 1);  // lands while this tile is being processed
      else
        load_tile(ktn);  // (converted into the other buffer after this tile's products)
    }
    const bf16* kb_lds = k_lds[kh][buf];
    const bf16* vb_lds = v_lds[kh][buf];
    const int cls = kt < kt_end ? cls_cur : kTileDead;  // a key half may sit out the last step
    if (cls != kTileDead) {
    const bool bias = MASK && (cls == kTileBias || a.alibi);  // add mask values and / or ALiBi
    const bool bits = MASK && cls == kTileBits;  // 0 / -inf block: use its visibility bits

    // S^T = K Q^T for both 32-key blocks; each K fragment serves all QB query blocks
    f32x16 st[QB][KB];
    #pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      #pragma unroll
      for (int kb = 0; kb < KB; ++kb) st[qb][kb] = zeros16();
    #pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      #pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 kf = TL::read_chunk(kb_lds, 32 * kb + r32, 2 * s + g);
        #pragma unroll
        for (int qb = 0; qb < QB; ++qb) mma(st[qb][kb], kf, qf[qb][s]);
      }
    }

    // does this tile need per-element masking (structure: sequence tail, causal diagonal,
    // lengths, window; or the block's bits)?
    const int key0 = kt * BN;
    const bool edge = !(key0 >= w_lo && key0 + BN <= w_hi);
    const bool masked = edge || bits;

    bf16x8 pf[QB][KB][2];
    #pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = qw + 32 * qb + r32;
      if (capped) {
        #pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(st[qb][kb][r] * cap_k);
            st[qb][kb][r] = cap_raw * (1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f));
          }
      }
      if (MASK && bias && a.alibi) {
        // ALiBi in raw score units: -(slope / scale) |key - position|; this lane's row, the
        // register's key: key - position = (key0 + 4 g - q_offset - row) + 32 kb + 8 rr + e
        const float sl = a.alibi[h] * args.inv_scale;
        const float base = (float)((int64_t)key0 + 4 * g - a.q_offset - row);
        #pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          #pragma unroll
          for (int r = 0; r < 16; ++r)
            st[qb][kb][r] -= sl * fabsf(base + (float)(32 * kb + 8 * (r >> 2) + (r & 3)));
      }
      if (MASK && bias && a.mask) {
        // the mask enters the raw score as M / scale so that one fma applies both later;
        // keys past the end read 0 (the tail is masked below), rows past the end the last row
        const float* mr = a.mask + b * a.mask_sb + h * a.mask_sh + (int64_t)min(row, a.Sq - 1) * a.mask_sq;
        #pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          #pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int k4 = key0 + 32 * kb + 8 * rr + 4 * g;  // 4 consecutive keys k4 .. k4 + 3
            float mv[4];
            if (k4 + 3 < a.Sk && args.mask_vec4) {
              const f32x4 m4 = *reinterpret_cast<const f32x4*>(mr + k4);
              mv[0] = m4[0]; mv[1] = m4[1]; mv[2] = m4[2]; mv[3] = m4[3];
            } else {
              #pragma unroll
              for (int e = 0; e < 4; ++e) mv[e] = (k4 + e < a.Sk) ? mr[k4 + e] : 0.f;
            }
            #pragma unroll
            for (int e = 0; e < 4; ++e) st[qb][kb][4 * rr + e] += mv[e] * args.inv_scale;
          }
        }
      }
      if (masked) {
        // keys of the tile this lane's row can see (bit j: key key0 + j); masked scores
        // become -inf (bit-field insert of -inf under a sign-extended bit: two VALU ops)
        int64_t lo, hi;
        key_range(a, klen, qlen, row, lo, hi);
        lo -= key0;
        hi -= key0;
        uint64_t vis = bit_range64((int)(lo < 0 ? 0 : (lo > BN ? BN : lo)), (int)(hi < 0 ? 0 : (hi > BN ? BN : hi)));
        if (bits) vis &= BN == 64 ? wb_cur[qb] : (wb_cur[qb] >> (key0 % kMaskTile));
        #pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const uint32_t wv = (uint32_t)(vis >> (32 * kb + 4 * g));  // bit 8 rr + e <-> register 4 rr + e
          #pragma unroll
          for (int r = 0; r < 16; ++r) st[qb][kb][r] = ninf_unless_bit(st[qb][kb][r], wv, 8 * (r >> 2) + (r & 3));
        }
      }
      // row max of this tile (raw score units), shared by lanes l and l ^ 32
      float mx = neg_inf();
      #pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        #pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(st[qb][kb][r], st[qb][kb][r + 1]));
      mx = halves_max(mx);
      const float mscaled = mx * cs;
      const bool need = mscaled > base[qb] + 8.f;
      if (__any(need)) {
        // lanes that keep their base use alpha = 1 (their base may still be -inf);
        // a lane moving off -inf gets alpha = 0, its accumulators being empty
        const float alpha = need ? fast_exp2(base[qb] - mscaled) : 1.f;
        const float nb = need ? mscaled : base[qb];
        base[qb] = nb;
        lsum[qb] *= alpha;
        #pragma unroll
        for (int db = 0; db < DB; ++db)
          #pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
      }
      const float nbase = (base[qb] == neg_inf()) ? 0.f : -base[qb];
      float ls = 0.f;
      #pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        #pragma unroll
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
    #pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int rbase = 32 * kb + 16 * hh + 4 * g + tr_row;
        #pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x4 lo = TL::read_tr(vb_lds, rbase, 32 * db + tr_col);
          const bf16x4 hi = TL::read_tr(vb_lds, rbase + 8, 32 * db + tr_col);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          #pragma unroll
          for (int qb = 0; qb < QB; ++qb) mma(oacc[qb][db], vf, pf[qb][kb][hh]);
        }
      }
    }

    }  // cls != dead
    if constexpr (KVF != 0) {
      if (more) commit_tile(buf ^ 1);
    }
    wait_vm();
    __syncthreads();
    #pragma unroll
    for (int j = 0; j < KS; ++j) tk[j] = tn[j];
    kt = ktn;
    cls_cur = cls_next;
    #pragma unroll
    for (int qb = 0; qb < QB; ++qb) wb_cur[qb] = wb_next[qb];
  }

  if constexpr (KS > 1) {
    // merge the key halves: half 1 leaves (base, sum, O) per lane in LDS (the tile buffers
    // are free after the last barrier), half 0 rescales both to the larger base and adds
    static_assert(KS == 2 && QB == 1, "the key split pairs two halves of one-block waves");
    constexpr int NV = DB * 16 + 2;  // floats per lane
    static_assert(RB * NV * 64 * 4 <= (int)sizeof(kv_lds), "merge buffer fits in the tile buffers");
    float* mrg = reinterpret_cast<float*>(&kv_lds[0][0][0][0]) + rb * NV * 64;
    if (kh == 1) {
      #pragma unroll
      for (int db = 0; db < DB; ++db)
        #pragma unroll
        for (int r = 0; r < 16; ++r) mrg[(db * 16 + r) * 64 + lane] = oacc[0][db][r];
      mrg[(DB * 16) * 64 + lane] = base[0];
      mrg[(DB * 16 + 1) * 64 + lane] = lsum[0];
    }
    __syncthreads();
    if (kh == 1) return;
    const float b1 = mrg[(DB * 16) * 64 + lane], l1 = mrg[(DB * 16 + 1) * 64 + lane];
    const float nb = fmaxf(base[0], b1);
    const float f0 = base[0] == neg_inf() ? 0.f : fast_exp2(base[0] - nb);
    const float f1 = b1 == neg_inf() ? 0.f : fast_exp2(b1 - nb);
    #pragma unroll
    for (int db = 0; db < DB; ++db)
      #pragma unroll
      for (int r = 0; r < 16; ++r) oacc[0][db][r] = oacc[0][db][r] * f0 + mrg[(db * 16 + r) * 64 + lane] * f1;
    lsum[0] = lsum[0] * f0 + l1 * f1;
    base[0] = nb;
  }

  if constexpr (SPLIT) {  // this share's normalised rows (bf16), their base and row sum, for the merge
    static_assert(QB == 1 && KS == 1, "the split walk runs the one-block, one-half configuration");
    const int row = qw + r32;
    const float lt = halves_sum(lsum[0]);
    const float inv = base[0] == neg_inf() ? 0.f : 1.f / lt;  // (a share that saw no key: zeros)
    if (row < a.Sq) {
      const int64_t r = (((int64_t)blockIdx.z * a.B + b) * a.Hq + h) * a.Sq + row;
      bf16* po = static_cast<bf16*>(args.part_o) + r * D;
      #pragma unroll
      for (int db = 0; db < DB; ++db)
        #pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 o4;
          #pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (bf16)(oacc[0][db][4 * rr + e] * inv);
          *reinterpret_cast<bf16x4*>(po + 32 * db + 8 * rr + 4 * g) = o4;
        }
      if (g == 0) *reinterpret_cast<float2*>(args.part_ml + 2 * r) = float2{base[0], lt};
    }
    return;
  }
  // epilogue: O = acc / l, LSE = (base + log2 l) ln 2; fully masked rows -> 0, 0. A sink
  // joins the row sum as 2^(sink log2e - base) after both move to the larger base (a row
  // with every key masked then keeps only the sink: O = 0, LSE = sink)
  const float sb = args.sinks ? args.sinks[h] * kLog2e : neg_inf();
  #pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw + 32 * qb + r32;
    float lt = halves_sum(lsum[qb]);
    float inv, lse;
    if (sb != neg_inf()) {
      const float nb = fmaxf(base[qb], sb);
      const float fo = base[qb] == neg_inf() ? 0.f : fast_exp2(base[qb] - nb);
      lt = lt * fo + fast_exp2(sb - nb);
      inv = fo / lt;
      lse = base[qb] == neg_inf() ? args.sinks[h] : (nb + log2f(lt)) * kLn2;
    } else {
      const bool full = base[qb] == neg_inf();
      inv = full ? 0.f : 1.f / lt;
      lse = full ? 0.f : (base[qb] + log2f(lt)) * kLn2;
    }
    if (row < a.Sq) {
      bf16* O = static_cast<bf16*>(args.o) + b * args.so.b + h * args.so.h + (int64_t)row * args.so.s;
      #pragma unroll
      for (int db = 0; db < DB; ++db) {
        #pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 o4;
          #pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (bf16)(oacc[qb][db][4 * rr + e] * inv);
          *reinterpret_cast<bf16x4*>(O + 32 * db + 8 * rr + 4 * g) = o4;
        }
      }
      if (g == 0) args.lse[b * args.lse_sb + h * args.lse_sh + row] = lse;
    }
  }
}

// Merge of a split forward: per row, each share's normalised row O_z (bf16) is weighted by
// its row sum rescaled to the largest base, w_z = l_z 2^(b_z - b), and O = sum w_z O_z /
// sum w_z, LSE = (b + log2 sum w_z) ln 2; a row no split
// saw a key for (every base -inf) gets O = 0, LSE = 0 (or LSE = its head's sink, which
// joins the row sum here). One pass over the splits with a
// running base (the online softmax's own rescale), one thread per 8 columns of a row; a
// workgroup takes 256 / (D / 8) rows of one (batch, head), with the first kMergeAhead shares'
// loads issued before any is used.
constexpr int kMergeAhead = 4;
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const FwdArgs args) {
  constexpr int TPR = D / 8;  // threads per row
  const AttnShape& a = args.a;
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const int h = blockIdx.y, b = blockIdx.z;
  const int i = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = 8 * (threadIdx.x % TPR);
  if (i >= a.Sq) return;
  const int64_t r = ((int64_t)b * a.Hq + h) * a.Sq + i;
  const int S = args.splits;
  float2 mls[kMergeAhead];
  bf16x8 p8s[kMergeAhead];
  #pragma unroll
  for (int z = 0; z < kMergeAhead; ++z) {
    if (z >= S) break;
    const int64_t zr = (int64_t)z * rows + r;
    mls[z] = *reinterpret_cast<const float2*>(args.part_ml + 2 * zr);
    p8s[z] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(args.part_o) + zr * D + c);
  }
  float mx = neg_inf(), l = 0.f;
  f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
  for (int z = 0; z < S; ++z) {
    float2 ml;
    bf16x8 p8;
    if (z < kMergeAhead) {
      #pragma unroll
      for (int y = 0; y < kMergeAhead; ++y)
        if (y == z) {
          ml = mls[y];
          p8 = p8s[y];
        }
    } else {
      const int64_t zr = (int64_t)z * rows + r;
      ml = *reinterpret_cast<const float2*>(args.part_ml + 2 * zr);
      p8 = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(args.part_o) + zr * D + c);
    }
    if (ml.x == neg_inf()) continue;  // this split saw no key of the row
    const float nm = fmaxf(mx, ml.x);
    // share z holds O_z = acc_z / l_z: its weight is l_z 2^(b_z - base)
    const float fo = mx == neg_inf() ? 0.f : fast_exp2(mx - nm), fn = fast_exp2(ml.x - nm) * ml.y;
    const f32x4 plo = {(float)p8[0], (float)p8[1], (float)p8[2], (float)p8[3]};
    const f32x4 phi = {(float)p8[4], (float)p8[5], (float)p8[6], (float)p8[7]};
    lo = lo * fo + plo * fn;
    hi = hi * fo + phi * fn;
    l = l * fo + fn;
    mx = nm;
  }
  float inv, lse;
  const float sb = args.sinks ? args.sinks[h] * kLog2e : neg_inf();
  if (sb != neg_inf()) {  // the sink joins the row sum at the larger of the two bases
    const float nb = fmaxf(mx, sb);
    const float fo = mx == neg_inf() ? 0.f : fast_exp2(mx - nb);
    l = l * fo + fast_exp2(sb - nb);
    inv = fo / l;
    lse = mx == neg_inf() ? args.sinks[h] : (nb + log2f(l)) * kLn2;
  } else {
    const bool full = mx == neg_inf();
    inv = full ? 0.f : 1.f / l;
    lse = full ? 0.f : (mx + log2f(l)) * kLn2;
  }
  bf16* O = static_cast<bf16*>(args.o) + b * args.so.b + h * args.so.h + (int64_t)i * args.so.s + c;
  *reinterpret_cast<bf16x8*>(O) = bf16x8{(bf16)(lo[0] * inv), (bf16)(lo[1] * inv), (bf16)(lo[2] * inv),
                                         (bf16)(lo[3] * inv), (bf16)(hi[0] * inv), (bf16)(hi[1] * inv),
                                         (bf16)(hi[2] * inv), (bf16)(hi[3] * inv)};
  if (c == 0) args.lse[b * args.lse_sb + h * args.lse_sh + i] = lse;
}

// stored fp16 / q8_0 K and V: the default walk without a dense mask or ALiBi (checked on the host)
template <int D, bool SPLIT>
hipError_t launch_kvf(const FwdArgs& args, dim3 grid, hipStream_t stream) {
  const bool causal = args.a.causal != 0, q8 = args.a.kvf == kKvQ8;
  if (causal && q8)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 64, true, false, 1, SPLIT, kKvQ8>), grid, dim3(256), 0, stream, args);
  else if (causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 64, true, false, 1, SPLIT, kKvF16>), grid, dim3(256), 0, stream, args);
  else if (q8)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 64, false, false, 1, SPLIT, kKvQ8>), grid, dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 64, false, false, 1, SPLIT, kKvF16>), grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const FwdArgs& args, hipStream_t stream) {
  const dim3 grid(args.a.Hq * args.a.B, (args.a.Sq + 127) / 128, args.splits);
  const bool causal = args.a.causal != 0, mask = args.a.mask != nullptr || args.a.alibi != nullptr;
  if (args.a.kvf != kKvBf16) {
    hipError_t e = launch_kvf<D, true>(args, grid, stream);
    if (e != hipSuccess) return e;
  } else if (causal && mask)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 64, true, true, 1, true>), grid, dim3(256), 0, stream, args);
  else if (causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 64, true, false, 1, true>), grid, dim3(256), 0, stream, args);
  else if (mask)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 64, false, true, 1, true>), grid, dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 64, false, false, 1, true>), grid, dim3(256), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows_per_wg = 256 / (D / 8);
  hipLaunchKernelGGL((fwd_merge_kernel<D>), dim3((args.a.Sq + rows_per_wg - 1) / rows_per_wg, args.a.Hq, args.a.B),
                     dim3(256), 0, stream, args);
  return hipGetLastError();
}

template <int D, int QB, int BN, int KS>
hipError_t launch_t(const FwdArgs& args, hipStream_t stream) {
  constexpr int BM = 4 / KS * QB * 32;
  const dim3 grid(args.a.Hq * args.a.B, (args.a.Sq + BM - 1) / BM);
  const bool causal = args.a.causal != 0, mask = args.a.mask != nullptr || args.a.alibi != nullptr;
  if (causal && mask)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BN, true, true, KS>), grid, dim3(256), 0, stream, args);
  else if (causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BN, true, false, KS>), grid, dim3(256), 0, stream, args);
  else if (mask)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BN, false, true, KS>), grid, dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BN, false, false, KS>), grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& args, int variant, hipStream_t stream) {
  if (args.a.kvf != kKvBf16)
    return launch_kvf<D, false>(args, dim3(args.a.Hq * args.a.B, (args.a.Sq + 127) / 128), stream);
  if (variant == 2) return launch_t<D, 2, 32, 1>(args, stream);
  if (variant == 3) return launch_t<D, 1, 32, 2>(args, stream);
  return launch_t<D, 1, 64, 1>(args, stream);
}

}  // namespace

// variant: 1 = 32 query rows per wave, 64-key tiles; 2 = 64 rows per wave, 32-key tiles;
// 3 = 32 rows per wave, keys split over two halves of the workgroup, 32-key tiles
hipError_t launch_fwd_bf16(const FwdArgs& args, int variant, hipStream_t stream) {
  return args.a.D == 64 ? launch_d<64>(args, variant, stream) : launch_d<128>(args, variant, stream);
}

hipError_t launch_fwd_bf16_split(const FwdArgs& args, hipStream_t stream) {
  return args.a.D == 64 ? launch_split_d<64>(args, stream) : launch_split_d<128>(args, stream);
}

}  // namespace fa
