// fa_api.hip -- the C ABI declared in include/fa_train.h: host-side argument
// checks, then kernel launches on the caller's stream. Nothing here allocates,
// synchronizes or reads device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "fa_kernels.h"
#include "fa_tile.h"
#include "fa_train.h"

namespace {

thread_local char g_err[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

struct Extent {
  uintptr_t lo, hi;  // byte range [lo, hi)
};

bool overlaps(const Extent& x, const Extent& y) { return x.lo < y.hi && y.lo < x.hi; }

// Checks one strided view of [B, H, S, W] elements of `elt` bytes (W contiguous).
// `align16` demands 16-byte aligned data and row strides; `out` demands that no two
// (b, h, s) rows overlap. Fills the byte extent for the alias checks.
fa_status check_view(const fa_view* v, const char* name, int64_t B, int64_t H, int64_t S, int64_t W, int elt,
                     bool align16, bool out, Extent* ext) {
  if (!v || !v->data) return fail(FA_ERR_NULL, "%s: view or data pointer is NULL", name);
  if (v->stride_b < 0 || v->stride_h < 0 || v->stride_s < 0)
    return fail(FA_ERR_STRIDE, "%s: negative stride", name);
  // the tile loads address a tile's rows with 32-bit byte offsets from the tile's start
  if (v->stride_s >= (int64_t(1) << 24))
    return fail(FA_ERR_STRIDE, "%s: stride_s (%lld) must be below 2^24 elements", name, (long long)v->stride_s);
  const uintptr_t base = reinterpret_cast<uintptr_t>(v->data);
  if (align16) {
    if (base % 16) return fail(FA_ERR_ALIGN, "%s: data pointer is not 16-byte aligned", name);
    if ((v->stride_b * elt) % 16 || (v->stride_h * elt) % 16 || (v->stride_s * elt) % 16)
      return fail(FA_ERR_ALIGN, "%s: strides must be multiples of 16 bytes", name);
  } else if (base % elt) {
    return fail(FA_ERR_ALIGN, "%s: data pointer is not %d-byte aligned", name, elt);
  }
  if (out) {
    // classic non-overlap test: sort the dims by stride, each stride must clear
    // the extent of the dims below it
    struct Dim {
      int64_t stride, n;
    } d[3] = {{v->stride_b, B}, {v->stride_h, H}, {v->stride_s, S}};
    std::sort(d, d + 3, [](const Dim& x, const Dim& y) { return x.stride < y.stride; });
    int64_t extent = W;
    for (int i = 0; i < 3; ++i) {
      if (d[i].n <= 1) continue;
      if (d[i].stride < extent) return fail(FA_ERR_STRIDE, "%s: output rows overlap", name);
      extent = d[i].stride * (d[i].n - 1) + extent;
    }
  }
  const int64_t last = (B - 1) * v->stride_b + (H - 1) * v->stride_h + (S - 1) * v->stride_s + W;
  ext->lo = base;
  ext->hi = base + (uintptr_t)(last * elt);
  return FA_OK;
}

fa_status check_params(const fa_attn_params* p) {
  if (!p) return fail(FA_ERR_NULL, "params pointer is NULL");
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Sq < 1 || p->Sk < 1 || p->D < 1)
    return fail(FA_ERR_SHAPE, "sizes must be positive (B=%d Hq=%d Hkv=%d Sq=%d Sk=%d D=%d)", p->B, p->Hq, p->Hkv,
                p->Sq, p->Sk, p->D);
  if (p->Hq % p->Hkv) return fail(FA_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->B > 65535 || p->Hq > 65535) return fail(FA_ERR_SHAPE, "B and Hq must be at most 65535");
  if (p->dtype != FA_F32 && p->dtype != FA_BF16) return fail(FA_ERR_DTYPE, "unknown dtype %d", p->dtype);
  if (p->D != 64 && p->D != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", p->D);
  if (p->causal != 0 && p->causal != 1) return fail(FA_ERR_SHAPE, "causal must be 0 or 1");
  if (p->q_offset < -(int64_t(1) << 40) || p->q_offset > (int64_t(1) << 40))
    return fail(FA_ERR_SHAPE, "q_offset out of range");
  if (!(p->scale > 0.f) || !isfinite(p->scale)) return fail(FA_ERR_SHAPE, "scale must be positive and finite");
  if (p->fwd_variant < 0 || p->fwd_variant > 3) return fail(FA_ERR_SHAPE, "unknown forward variant %d", p->fwd_variant);
  if (p->q_split_tiles < 0) return fail(FA_ERR_SHAPE, "q_split_tiles must be >= 0");
  if (p->bwd_kv_walk < 0 || p->bwd_kv_walk > 2) return fail(FA_ERR_SHAPE, "bwd_kv_walk %d (0, 1 or 2)", p->bwd_kv_walk);
  if (p->kv_format < FA_KV_DTYPE || p->kv_format > FA_KV_Q8_0)
    return fail(FA_ERR_DTYPE, "unknown kv_format %d", p->kv_format);
  if (p->kv_format != FA_KV_DTYPE) {
    if (p->dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "stored K / V formats need bf16 problems");
    if (p->mask || p->alibi || p->softcap != 0.f)
      return fail(FA_ERR_UNSUPPORTED, "stored K / V formats take no dense mask, ALiBi or softcap");
  }
  if (p->kv_split < 0 || p->kv_split > 64 || p->q_split < 0 || p->q_split > 64 || p->fwd_split < 0 ||
      p->fwd_split > 64)
    return fail(FA_ERR_SHAPE, "split hints must be in 0 .. 64");
  if (p->window_left < -1 || p->window_right < -1) return fail(FA_ERR_SHAPE, "window bounds must be >= -1");
  if (reinterpret_cast<uintptr_t>(p->sinks) % 4) return fail(FA_ERR_ALIGN, "sinks is not 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(p->alibi) % 4) return fail(FA_ERR_ALIGN, "alibi is not 4-byte aligned");
  if (p->bwd_dq_launch < 0 || p->bwd_dq_launch > 4)
    return fail(FA_ERR_SHAPE, "bwd_dq_launch must be 0 to 4 (got %d)", p->bwd_dq_launch);
  if (reinterpret_cast<uintptr_t>(p->key_len) % 4 || reinterpret_cast<uintptr_t>(p->q_len) % 4)
    return fail(FA_ERR_ALIGN, "key_len / q_len are not 4-byte aligned");
  if (!(p->softcap >= 0.f) || isinf(p->softcap)) return fail(FA_ERR_SHAPE, "softcap must be >= 0 and finite");
  if (p->dbias) {
    if (!p->mask) return fail(FA_ERR_SHAPE, "dbias is the gradient of a dense mask: mask is NULL");
    if (p->dtype == FA_BF16 && p->softcap > 0.f)
      return fail(FA_ERR_UNSUPPORTED, "the mask gradient is not produced under a logit softcap in bf16");
    if (p->dbias_stride_b < 0 || p->dbias_stride_h < 0 || p->dbias_stride_q < p->Sk)
      return fail(FA_ERR_STRIDE, "dbias strides must be >= 0 with dbias_stride_q >= Sk");
    if (p->B > 1 && (p->dbias_stride_b == 0) != (p->mask_stride_b == 0))
      return fail(FA_ERR_STRIDE, "dbias must be shared by the batch exactly when the mask is");
    if (p->Hq > 1 && (p->dbias_stride_h == 0) != (p->mask_stride_h == 0))
      return fail(FA_ERR_STRIDE, "dbias must be shared by the heads exactly when the mask is");
    if (reinterpret_cast<uintptr_t>(p->dbias) % 4) return fail(FA_ERR_ALIGN, "dbias is not 4-byte aligned");
  }
  if (p->mask) {
    if (p->mask_stride_q < p->Sk) return fail(FA_ERR_STRIDE, "mask_stride_q (%lld) < Sk", (long long)p->mask_stride_q);
    if (p->mask_stride_b < 0) return fail(FA_ERR_STRIDE, "mask_stride_b is negative");
    if (p->mask_stride_h < 0) return fail(FA_ERR_STRIDE, "mask_stride_h is negative");
    if (p->mask_stride_h > 0 && p->mask_tiles)
      return fail(FA_ERR_UNSUPPORTED, "the mask block map is per batch entry: a mask per head runs without one");
    if (reinterpret_cast<uintptr_t>(p->mask) % 4) return fail(FA_ERR_ALIGN, "mask pointer is not 4-byte aligned");
  }
  return FA_OK;
}

Extent mask_extent(const fa_attn_params* p) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(p->mask);
  const int64_t last = (int64_t)(p->B - 1) * p->mask_stride_b + (int64_t)(p->Hq - 1) * p->mask_stride_h +
                       (int64_t)(p->Sq - 1) * p->mask_stride_q + p->Sk;
  return {base, base + (uintptr_t)(last * 4)};
}

int64_t tile_rows(const fa_attn_params* p) { return (p->Sq + 63) / 64; }
int64_t tile_cols(const fa_attn_params* p) { return (p->Sk + 63) / 64; }
int64_t tile_batches(const fa_attn_params* p) { return p->mask_stride_b == 0 ? 1 : p->B; }

fa::AttnShape shape_of(const fa_attn_params* p) {
  fa::AttnShape a;
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.Sq = p->Sq;
  a.Sk = p->Sk;
  a.D = p->D;
  a.G = p->Hq / p->Hkv;
  a.causal = p->causal;
  a.q_offset = p->q_offset;
  a.scale = p->scale;
  a.mask = p->mask;
  a.mask_sb = p->mask_stride_b;
  a.mask_sq = p->mask_stride_q;
  a.mask_sh = p->mask ? p->mask_stride_h : 0;
  a.tiles = p->mask ? p->mask_tiles : nullptr;
  const int64_t nblk = tile_batches(p) * tile_rows(p) * tile_cols(p);
  const int64_t rowbits_off = (nblk + 255) / 256 * 256;
  a.rowbits = a.tiles ? reinterpret_cast<const uint64_t*>(a.tiles + rowbits_off) : nullptr;
  a.colbits = a.tiles ? a.rowbits + nblk * 64 : nullptr;
  a.tiles_ncol = (int)tile_cols(p);
  a.tiles_bstride = p->mask_stride_b == 0 ? 0 : (int)(tile_rows(p) * tile_cols(p));
  a.key_len = p->key_len;
  a.q_len = p->q_len;
  a.wl = p->window_left;
  a.wr = p->window_right;
  a.alibi = p->alibi;
  a.softcap = p->softcap;
  a.kvf = p->kv_format == FA_KV_F16 ? fa::kKvF16 : p->kv_format == FA_KV_Q8_0 ? fa::kKvQ8 : fa::kKvBf16;
  const bool q8 = p->kv_format == FA_KV_Q8_0;
  a.kscale = q8 ? static_cast<const _Float16*>(p->k_scale.data) : nullptr;
  a.vscale = q8 ? static_cast<const _Float16*>(p->v_scale.data) : nullptr;
  a.sks = q8 ? fa::Strides{p->k_scale.stride_b, p->k_scale.stride_h, p->k_scale.stride_s} : fa::Strides{0, 0, 0};
  a.svs = q8 ? fa::Strides{p->v_scale.stride_b, p->v_scale.stride_h, p->v_scale.stride_s} : fa::Strides{0, 0, 0};
  return a;
}

// Bytes per stored K / V element, and the checks of the K / V views and (q8_0) their scale
// planes; `ins` receives their extents for the alias checks.
int kv_elt(const fa_attn_params* p) {
  return p->kv_format == FA_KV_Q8_0 ? 1 : p->kv_format == FA_KV_F16 ? 2 : (p->dtype == FA_BF16 ? 2 : 4);
}
fa_status check_kv(const fa_attn_params* p, const fa_view* k, const fa_view* v, Extent* ins, int* n_in,
                   const char** in_names) {
  fa_status s;
  const int e = kv_elt(p);
  Extent ek, ev;
  if ((s = check_view(k, "k", p->B, p->Hkv, p->Sk, p->D, e, true, false, &ek))) return s;
  if ((s = check_view(v, "v", p->B, p->Hkv, p->Sk, p->D, e, true, false, &ev))) return s;
  ins[*n_in] = ek;
  in_names[(*n_in)++] = "k";
  ins[*n_in] = ev;
  in_names[(*n_in)++] = "v";
  if (p->kv_format == FA_KV_Q8_0) {
    Extent eks, evs;
    if ((s = check_view(&p->k_scale, "k_scale", p->B, p->Hkv, p->Sk, p->D / 32, 2, false, false, &eks))) return s;
    if ((s = check_view(&p->v_scale, "v_scale", p->B, p->Hkv, p->Sk, p->D / 32, 2, false, false, &evs))) return s;
    if (p->Sk > 1 && (p->k_scale.stride_s < p->D / 32 || p->v_scale.stride_s < p->D / 32))
      return fail(FA_ERR_STRIDE, "k_scale / v_scale: stride_s must cover a row's D / 32 scales");
    ins[*n_in] = eks;
    in_names[(*n_in)++] = "k_scale";
    ins[*n_in] = evs;
    in_names[(*n_in)++] = "v_scale";
  }
  return FA_OK;
}

// The generic backward (fa_bwd.hip) runs fp32 problems and logit softcaps over a dense
// mask; the bf16 MFMA backward runs the rest (a softcap without a dense mask in a variant of
// its own). The bf16 forward takes every softcap itself.
// the backward's generic kernels: the fp32 problems (bf16 runs on the matrix-core walks)
bool generic_path(const fa_attn_params* p) { return p->dtype != FA_BF16; }

fa::Strides strides_of(const fa_view* v) { return {v->stride_b, v->stride_h, v->stride_s}; }

int elt_of(const fa_attn_params* p) { return p->dtype == FA_BF16 ? 2 : 4; }

fa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

fa_status check_alias(const Extent* outs, int n_out, const char* const* out_names, const Extent* ins, int n_in,
                      const char* const* in_names) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], ins[j]))
        return fail(FA_ERR_ALIAS, "output %s overlaps input %s", out_names[i], in_names[j]);
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], outs[j]))
        return fail(FA_ERR_ALIAS, "outputs %s and %s overlap", out_names[i], out_names[j]);
  }
  return FA_OK;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Split factors of the bf16 backward. Each split > 1 spreads one tile's walk over
// several workgroups, each storing its fp32 partial sums into a slice of its own in the
// workspace; a reduce pass then sums the slices. Splits are only used when the unsplit
// grid would leave compute units idle.
// Predicted time (us) of the bf16 backward for one split choice. The workgroups are
// taken in dispatch order (dK/dV units by key tile, longest causal walks first, then
// dQ units, longest first), each costed by its walk length, and placed greedily on
// the compute units the way the dispatcher fills whichever frees first; split
// choices add the reduce pass over their fp32 slices.
double predict_bwd_us(const fa_attn_params* p, int kv, int q, int64_t q_tiles) {
  // fitted to MI355X timings of the three bf16 workloads over the split grid
  constexpr double kPairUs = 2.7;         // one 64-row x 128-key dK/dV step
  constexpr double kTileUs = 1.8;         // one 128-row x 64-key dQ step
  constexpr double kKvUnitUs = 8.0;       // a dK/dV workgroup's first loads and its stores
  constexpr double kPassUs = 4.0;         // one more kernel on the stream
  constexpr double kBytesPerUs = 5.0e6;   // streaming rate of the reduce pass
  const int U = fa::kBwdUnit, slots = 1024 / fa::kBwdWaves;
  const int64_t nkt = (p->Sk + U - 1) / U, nqt = (p->Sq + U - 1) / U;
  const int64_t nr64 = (p->Sq + 63) / 64, nk64 = (p->Sk + 63) / 64;
  const int G = p->Hq / p->Hkv;
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < slots; ++i) free_at.push(0.0);
  double end = 0.0;
  auto place = [&](double cost) {
    const double t = free_at.top() + cost;
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  };
  for (int64_t kt = 0; kt < nkt; ++kt) {
    int64_t qt0 = 0;  // first 64-row tile that sees this key tile
    if (p->causal) {
      const int64_t first_row = kt * U - p->q_offset;
      qt0 = first_row <= 0 ? 0 : std::min<int64_t>(first_row / 64, nr64);
    }
    const int64_t pairs = G * (nr64 - qt0);
    const double cost = kKvUnitUs + kPairUs * (double)((pairs + kv - 1) / kv);
    for (int64_t u = 0; u < (int64_t)p->B * p->Hkv * kv; ++u) place(cost);
  }
  // whole query tiles first, then the q_tiles first tiles split q ways
  if (q <= 1) q_tiles = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t lo = pass == 0 ? q_tiles : 0, hi = pass == 0 ? nqt : q_tiles;
    const int ways = pass == 0 ? 1 : q;
    for (int64_t qt = hi - 1; qt >= lo; --qt) {
      int64_t tiles = nk64;
      if (p->causal) {
        const int64_t last_key = p->q_offset + (qt + 1) * U - 1;
        tiles = last_key < 0 ? 0 : std::min<int64_t>(last_key / 64 + 1, nk64);
      }
      const double cost = kTileUs * (double)((tiles + ways - 1) / ways);
      for (int64_t u = 0; u < (int64_t)p->B * p->Hq * ways; ++u) place(cost);
    }
  }
  const double nk = (double)p->B * p->Hkv * p->Sk * p->D, nq = (double)p->B * p->Hq * p->Sq * p->D;
  if (kv > 1) end += kPassUs + (2.0 * kv * nk * 4.0 + 2.0 * nk * 2.0) / kBytesPerUs;
  if (q > 1 && q_tiles > 0) {
    const double rows = std::min<double>(1.0, (double)(q_tiles * U) / p->Sq);  // share of rows reduced
    end += kPassUs + rows * (q * nq * 4.0 + nq * 2.0) / kBytesPerUs;
  }
  return end;
}

// Split choice of the bf16 backward: the candidate with the least predicted time, kept
// per shape in a small per-thread cache (the prediction walks every workgroup). Calls
// with the same shape always get the same choice, so the workspace size the caller
// was given matches the launch.
void choose_splits(const fa_attn_params* p, bool accumulate, int* kv_split, int* q_split, int* q_tiles_split) {
  (void)accumulate;
  const int64_t nqt = (p->Sq + fa::kBwdUnit - 1) / fa::kBwdUnit;
  int kv = 1, q = 1, qt = 0;
  const int64_t units = (int64_t)((p->Sk + fa::kBwdUnit - 1) / fa::kBwdUnit) * p->B * p->Hkv + nqt * p->B * p->Hq;
  if (units < 8 * 1024) {
    struct Entry {
      int64_t key[8];
      int kv, q, qt;
    };
    thread_local Entry cache[16];
    thread_local int next = 0;
    const int64_t key[8] = {p->B, p->Hq, p->Hkv, p->Sq, p->Sk, p->D, p->causal, p->q_offset};
    bool hit = false;
    for (const Entry& e : cache)
      if (e.kv > 0 && std::equal(key, key + 8, e.key)) {
        kv = e.kv;
        q = e.q;
        qt = e.qt;
        hit = true;
        break;
      }
    const int64_t kv_units = (int64_t)((p->Sk + fa::kBwdUnit - 1) / fa::kBwdUnit) * p->B * p->Hkv;
    const int64_t q_units = nqt * p->B * p->Hq;
    if (!hit && !p->causal && p->window_left < 0 && p->window_right < 0) {
      // Without a causal diagonal or a window every unit of a kind has about the same walk, and
      // the cost model below ranks the splits of such grids poorly (it preferred splits that
      // measured 6-17% slower). Measured on MI355X (DiT self-attention, its key-length form and
      // DiT cross-attention, graph replays): the dK/dV walks split two ways when their grid is at
      // most one workgroup per compute unit, and the dQ walks of the first half of the query
      // tiles (dispatched last) split two ways when the dQ grid is that small too. (Under a
      // 256-key band the walks are short and the same rule measured 15% slower than the model's
      // choice.)
      const int64_t kv_walk = (int64_t)((p->Sq + 63) / 64) * (p->Hq / p->Hkv), q_walk = (p->Sk + 63) / 64;
      kv = kv_units <= 256 && kv_walk >= 2 ? 2 : 1;
      if (q_units < 256 && nqt >= 2 && q_walk >= 2) {
        q = 2;
        qt = (int)(nqt / 2);
      }
      hit = true;
    }
    if (!hit) {
      const int64_t kv_pairs = (int64_t)((p->Sq + 63) / 64) * (p->Hq / p->Hkv);  // walk length, one key tile
      const int64_t q_walk = (p->Sk + 63) / 64;                                   // walk length, one query tile
      // split query tiles: all of them. (Splitting only the first ones, dispatched last, is
      // left to the q_split_tiles hint: it shortened the DiT self-attention backward by
      // 10% on MI355X, but this dispatch-order model does not rank those choices reliably:
      // it preferred four-way tails that measured 17% slower.)
      const int64_t step = nqt;
      double best = predict_bwd_us(p, 1, 1, 0);
      for (int ckv : {1, 2, 4, 8})
        for (int cq : {1, 2, 4, 8, 16}) {
          if (ckv > std::max<int64_t>(kv_pairs, 1) || cq > std::max<int64_t>(q_walk, 1)) continue;
          for (int64_t ct = cq > 1 ? step : 0; ct <= (cq > 1 ? nqt : 0); ct += (cq > 1 ? step : 1)) {
            const int64_t tiles = cq > 1 && ct + step > nqt ? nqt : ct;  // (the last step takes them all)
            if (ckv == 1 && cq == 1) continue;
            const double t = predict_bwd_us(p, ckv, cq, tiles);
            if (t < 0.98 * best) {  // a split must pay for itself clearly
              best = t;
              kv = ckv;
              q = cq;
              qt = (int)tiles;
            }
            if (cq == 1) break;
          }
        }
      Entry& e = cache[next];
      next = (next + 1) % 16;
      std::copy(key, key + 8, e.key);
      e.kv = kv;
      e.q = q;
      e.qt = qt;
    }
  }
  *kv_split = p->kv_split ? p->kv_split : kv;
  if (p->q_split) {  // given: all query tiles, or the q_split_tiles first ones
    *q_split = p->q_split;
    *q_tiles_split = (int)(p->q_split_tiles ? std::min<int64_t>(p->q_split_tiles, nqt) : nqt);
  } else {
    *q_split = q;
    *q_tiles_split = p->q_split_tiles && q > 1 ? (int)std::min<int64_t>(p->q_split_tiles, nqt) : qt;
  }
  if (*q_split <= 1) *q_tiles_split = 0;
}

struct WsLayout {
  size_t dq_off, dk_off, dv_off, ds_off, total;
  bool need_dq, need_dkdv, need_ds;
};

// Does the bf16 backward take dQ from the dS the dK/dV walk stores (instead of the dQ walk
// recomputing S and dP)? When asked (bwd_dq_launch 3), or automatically (0) for a dQ grid of
// at least 512 128-row workgroups (measured on MI355X over graph replays: the causal LM layer,
// 1024 workgroups, gains 3% plain, 4-6% with ALiBi or a softcap; the DiT workloads, 208 to 416,
// gain nothing, their dQ walk filling the compute units the dK/dV walk leaves idle), except
// for callers that cannot allocate (the static scratch is too small to hold dS). Never for a
// stored K/V window, the mask's gradient (added by the dQ walk) or the role-split dK/dV walk.
size_t ds_bytes(const fa_attn_params* p) {
  return (size_t)p->B * p->Hq * ((p->Sq + 63) / 64) * ((p->Sk + fa::kBwdUnit - 1) / fa::kBwdUnit) * fa::kDsBlock;
}
// (the automatic choice also keeps the stored dS within 2 GB of workspace: one block per
// (head, 64-row tile, 128-key tile), causal or not)
constexpr size_t kAutoDsBytes = size_t(2) << 30;
bool dq_from_ds(const fa_attn_params* p, bool noalloc = false) {
  if (generic_path(p) || p->kv_format != FA_KV_DTYPE || p->dbias || p->bwd_kv_walk == 2) return false;
  if (p->bwd_dq_launch == 3) return true;
  if (p->bwd_dq_launch != 0 || noalloc) return false;
  return (int64_t)((p->Sq + fa::kBwdUnit - 1) / fa::kBwdUnit) * p->B * p->Hq >= 512 && ds_bytes(p) <= kAutoDsBytes;
}

// Workspace of the backward: the fp32 partial slices of the chosen split (bf16), or the
// fp32 dQ accumulator (fp32 inputs).
WsLayout workspace_layout(const fa_attn_params* p, bool accumulate, bool noalloc = false) {
  WsLayout w;
  const size_t nq = (size_t)p->B * p->Hq * p->Sq * p->D * sizeof(float);
  const size_t nk = (size_t)p->B * p->Hkv * p->Sk * p->D * sizeof(float);
  size_t dq_bytes = nq, dk_bytes = 0;
  if (!generic_path(p)) {
    int kv, q, qt;
    choose_splits(p, accumulate, &kv, &q, &qt);
    w.need_dq = q > 1 && qt > 0;
    w.need_dkdv = kv > 1;
    dq_bytes = w.need_dq ? q * nq : 0;
    dk_bytes = w.need_dkdv ? kv * nk : 0;
  } else {
    w.need_dq = true;
    w.need_dkdv = false;
  }
  w.need_ds = dq_from_ds(p, noalloc);
  w.dq_off = 0;
  w.dk_off = w.need_dq ? round256(dq_bytes) : 0;
  w.dv_off = w.dk_off + (w.need_dkdv ? round256(dk_bytes) : 0);
  w.ds_off = w.dv_off + (w.need_dkdv ? round256(dk_bytes) : 0);
  w.total = w.ds_off + (w.need_ds ? round256(ds_bytes(p)) : 0);
  return w;
}

size_t workspace_bytes(const fa_attn_params* p) { return workspace_layout(p, false).total; }

// Scratch memory of fa_train_bwd_noalloc, for callers that cannot allocate: the
// workspace of the backward (split walks' fp32 slices, or the fp32 path's dQ
// accumulator) lives in this static device array instead of a caller-owned buffer.
// Every device the library runs on holds its own copy until the process ends. In host
// code `scratch` names a host-side stand-in, not the device copy: the device address
// is looked up once per device with hipGetSymbolAddress and only that address is ever
// handed to kernels.
static __device__ __align__(256) char scratch[FA_TRAIN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first call on
// that device, with it current).
fa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_HIP, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// A second stream per device for the dQ kernel that runs beside the dK/dV kernel, with the two
// events that fork it from the caller's stream and join it back. Created on first use (default
// priority); the mutex makes each call's record / wait / launch sequence atomic, so calls from
// several host threads cannot join on each other's events.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
SideStream g_side[kMaxDevices];
std::mutex g_side_init_mu;

fa_status side_of_current_device(SideStream** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_HIP, "device %d beyond the stream table", dev);
  std::lock_guard<std::mutex> lock(g_side_init_mu);
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess ||
        (e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess)
      return fail(FA_ERR_HIP, "creating the dQ stream on device %d: %s", dev, hipGetErrorString(e));
  }
  *out = &ss;
  return FA_OK;
}

#ifdef FA_CHECK
struct Checker {
  char* msg;
  size_t len;
  bool ok = true;
  void fail(const char* fmt, ...) {
    if (!ok) return;
    ok = false;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, len, fmt, ap);
    va_end(ap);
  }
};

void check_bwd(Checker& c, const fa_attn_params* p, const int32_t* klen_h, const int32_t* qlen_h);
void check_fwd(Checker& c, const fa_attn_params* p, const int32_t* klen_h, const int32_t* qlen_h);
#endif

// Shared body of the backward entry points. use_scratch: the workspace is the current
// device's static scratch array (fa_train_bwd_noalloc), looked up after every host check.
fa_status bwd_common(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                     const fa_view* dout, const fa_view* lse, const fa_view* delta, const fa_view* dq,
                     const fa_view* dk, const fa_view* dv, void* workspace, size_t workspace_bytes_given,
                     hipStream_t stream, bool accumulate, bool use_scratch = false) {
  fa_status s = check_params(p);
  if (s) return s;
  const int elt = elt_of(p);
  Extent eq, edo, el, ed, edq, edk, edv;
  Extent kvx[4];
  const char* kv_names[4];
  int n_kv = 0;
  if ((s = check_view(q, "q", p->B, p->Hq, p->Sq, p->D, elt, true, false, &eq))) return s;
  if ((s = check_kv(p, k, v, kvx, &n_kv, kv_names))) return s;
  if ((s = check_view(dout, "dout", p->B, p->Hq, p->Sq, p->D, elt, true, false, &edo))) return s;
  if (!lse || !delta) return fail(FA_ERR_NULL, "lse or delta view is NULL");
  if (lse->stride_s != 1 || delta->stride_s != 1) return fail(FA_ERR_STRIDE, "lse / delta stride_s must be 1");
  if ((s = check_view(lse, "lse", p->B, p->Hq, p->Sq, 1, 4, false, false, &el))) return s;
  if ((s = check_view(delta, "delta", p->B, p->Hq, p->Sq, 1, 4, false, false, &ed))) return s;
  if ((s = check_view(dq, "dq", p->B, p->Hq, p->Sq, p->D, elt, true, true, &edq))) return s;
  const int gelt = accumulate ? 4 : elt;
  if ((s = check_view(dk, accumulate ? "dk_acc" : "dk", p->B, p->Hkv, p->Sk, p->D, gelt, true, true, &edk))) return s;
  if ((s = check_view(dv, accumulate ? "dv_acc" : "dv", p->B, p->Hkv, p->Sk, p->D, gelt, true, true, &edv))) return s;
  const WsLayout wl = workspace_layout(p, accumulate, use_scratch);
  const size_t need = wl.total;
  if (use_scratch) {
    if (need > (size_t)FA_TRAIN_NOALLOC_SCRATCH_BYTES)
      return fail(FA_ERR_WORKSPACE, "this backward needs %zu bytes of scratch; the static array holds %zu",
                  need, (size_t)FA_TRAIN_NOALLOC_SCRATCH_BYTES);
  } else if (need > 0) {
    if (!workspace) return fail(FA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes_given < need)
      return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_given, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(FA_ERR_ALIGN, "workspace is not 256-byte aligned");
  }
  const uintptr_t wlo = reinterpret_cast<uintptr_t>(workspace);
  Extent ews = {wlo, use_scratch ? wlo : wlo + need};  // (the static array is nobody else's memory)
  Extent ins[10] = {eq, edo, el, ed};
  const char* in_names[10] = {"q", "dout", "lse", "delta"};
  int n_in = 4;
  for (int i = 0; i < n_kv; ++i) {
    in_names[n_in] = kv_names[i];
    ins[n_in++] = kvx[i];
  }
  if (p->mask) {
    in_names[n_in] = "mask";
    ins[n_in++] = mask_extent(p);
  }
  Extent outs[5] = {edq, edk, edv, ews};
  const char* out_names[5] = {"dq", accumulate ? "dk_acc" : "dk", accumulate ? "dv_acc" : "dv", "workspace", "dbias"};
  int n_out = 4;
  if (p->dbias) {  // rows of Sk fp32 entries, one plane per batch entry / head unless shared
    const fa_view dbv = {p->dbias, p->dbias_stride_b, p->dbias_stride_h, p->dbias_stride_q};
    if ((s = check_view(&dbv, "dbias", p->dbias_stride_b ? p->B : 1, p->dbias_stride_h ? p->Hq : 1, p->Sq, p->Sk, 4,
                        false, true, &outs[n_out++])))
      return s;
  }
  if ((s = check_alias(outs, n_out, out_names, ins, n_in, in_names))) return s;
  if (use_scratch && need > 0) {
    if ((s = scratch_of_current_device(&workspace))) return s;
    workspace_bytes_given = FA_TRAIN_NOALLOC_SCRATCH_BYTES;
  }

#ifdef FA_CHECK
  if (!generic_path(p)) {  // the checked build verifies the launch's index space first
    char rep[256];
    Checker c{rep, sizeof rep};
    check_bwd(c, p, nullptr, nullptr);
    if (!c.ok) return fail(FA_ERR_HIP, "FA_CHECK: %s", rep);
  }
#endif
  fa::BwdArgs a;
  a.a = shape_of(p);
  a.q = q->data;
  a.k = k->data;
  a.v = v->data;
  a.dout = dout->data;
  a.lse = static_cast<const float*>(lse->data);
  a.delta = static_cast<const float*>(delta->data);
  a.dk = dk->data;
  a.dv = dv->data;
  a.sq = strides_of(q);
  a.sk = strides_of(k);
  a.sv = strides_of(v);
  a.sdo = strides_of(dout);
  a.sdk = strides_of(dk);
  a.sdv = strides_of(dv);
  a.lse_sb = lse->stride_b;
  a.lse_sh = lse->stride_h;
  a.delta_sb = delta->stride_b;
  a.delta_sh = delta->stride_h;
  a.accumulate = accumulate ? 1 : 0;
  a.inv_scale = 1.f / p->scale;
  a.dbias = p->dbias;
  a.dbias_sb = p->dbias_stride_b;
  a.dbias_sh = p->dbias_stride_h;
  a.dbias_sq = p->dbias_stride_q;
  a.dbias_atomic = (p->B > 1 && p->dbias_stride_b == 0) || (p->Hq > 1 && p->dbias_stride_h == 0);
  a.dbias_vec4 = reinterpret_cast<uintptr_t>(p->dbias) % 16 == 0 && p->dbias_stride_b % 4 == 0 &&
                 p->dbias_stride_h % 4 == 0 && p->dbias_stride_q % 4 == 0;
  const uintptr_t mp = reinterpret_cast<uintptr_t>(p->mask);
  a.mask_vec4 = p->mask && mp % 16 == 0 && p->mask_stride_q % 4 == 0 && p->mask_stride_b % 4 == 0 &&
                 p->mask_stride_h % 4 == 0;
  const int is_bf16 = p->dtype == FA_BF16;
  fa_status st;
  if (!generic_path(p)) {
    char* ws = static_cast<char*>(workspace);
    fa::BwdPlan plan;
    int kv, q, qt;
    choose_splits(p, accumulate, &kv, &q, &qt);
    // the one-wave dK/dV walk unless the hint asks for the role-split one (which has no
    // softcap variant): measured on MI355X, the role-split walk waits on its barriers and P
    // hand-over 55% of the time and stages a pair's tiles per 64 keys instead of 128, and was
    // 20-60% slower on the DiT and LM workloads
    const int kv_role = p->softcap > 0.f || p->kv_format != FA_KV_DTYPE ? 0 : (p->bwd_kv_walk == 2 ? 1 : 0);
    fa::plan_bwd_bf16(a.a, kv, q, qt, 0, &plan, kv_role, wl.need_ds ? 1 : 0);
    // a large dQ grid runs as its own kernel, two workgroups per compute unit (measured on
    // the causal LM backward: 659 -> 631 us); small grids keep one launch, whose dQ
    // workgroups fill the compute units the dK/dV walks leave idle
    plan.dq_separate = p->bwd_dq_launch ? p->bwd_dq_launch >= 2 : plan.n_q_units >= 512;
    // the separate dQ kernel on a second stream, beside the dK/dV kernel (not for callers that
    // cannot allocate, and not over stored dS, which the dQ pass reads after the walk)
    const bool beside = !use_scratch && p->bwd_dq_launch == 4 && !wl.need_ds && plan.n_kv_units > 0 &&
                        plan.n_q_units > 0;
    // split walks write every element of their fp32 slices (zeros included), so the
    // slices need no clearing; the reduce passes sum them into the outputs
    a.dq_acc = nullptr;
    plan.dq_part = wl.need_dq ? reinterpret_cast<float*>(ws + wl.dq_off) : nullptr;
    plan.dk_part = wl.need_dkdv ? reinterpret_cast<float*>(ws + wl.dk_off) : nullptr;
    plan.dv_part = wl.need_dkdv ? reinterpret_cast<float*>(ws + wl.dv_off) : nullptr;
    plan.dq = dq->data;
    plan.sdq = strides_of(dq);
    if (wl.need_ds) plan.ds = ws + wl.ds_off;
    const int64_t nq = (int64_t)p->B * p->Hq * p->Sq * p->D, nk = (int64_t)p->B * p->Hkv * p->Sk * p->D;
    if (beside) {
      SideStream* ss = nullptr;
      if ((st = side_of_current_device(&ss))) return st;
      std::lock_guard<std::mutex> lock(ss->mu);
      if ((st = hip_status(hipEventRecord(ss->fork, stream), "dQ stream fork")) ||
          (st = hip_status(hipStreamWaitEvent(ss->s, ss->fork, 0), "dQ stream fork")))
        return st;
      plan.dq_stream = ss->s;
      if ((st = hip_status(fa::launch_bwd_bf16(a, plan, stream), "backward"))) return st;
      if ((st = hip_status(hipEventRecord(ss->join, ss->s), "dQ stream join")) ||
          (st = hip_status(hipStreamWaitEvent(stream, ss->join, 0), "dQ stream join")))
        return st;
    } else if ((st = hip_status(fa::launch_bwd_bf16(a, plan, stream), "backward"))) {
      return st;
    }
    // the reduce passes: dQ over the rows of the split query tiles (the first ones), dK and dV
    // over every key; one launch when all three go to bf16 outputs (the chunked walk adds dK / dV
    // into its fp32 window accumulators instead)
    const int rows = std::min(p->Sq, plan.q_tiles_split * plan.q_bm);
    const fa::ReduceArgs r = {p->B, p->Hq, rows, p->D, p->Sq, plan.dq_part, q, nq, dq->data, strides_of(dq),
                              p->scale, 0};
    const int out_bf16 = accumulate ? 0 : 1, acc = accumulate ? 1 : 0;
    const fa::ReduceArgs rk = {p->B, p->Hkv, p->Sk, p->D, p->Sk, plan.dk_part, kv, nk,
                               dk->data, strides_of(dk), p->scale, acc};
    const fa::ReduceArgs rv = {p->B, p->Hkv, p->Sk, p->D, p->Sk, plan.dv_part, kv, nk,
                               dv->data, strides_of(dv), 1.f, acc};
    if (wl.need_dq && wl.need_dkdv && !accumulate) {
      if ((st = hip_status(fa::launch_reduce_parts(rk, &rv, &r, 1, stream), "dq / dk / dv reduce"))) return st;
    } else {
      if (wl.need_dq && (st = hip_status(fa::launch_reduce_parts(r, nullptr, nullptr, 1, stream), "dq reduce")))
        return st;
      if (wl.need_dkdv &&
          (st = hip_status(fa::launch_reduce_parts(rk, &rv, nullptr, out_bf16, stream), "dk / dv reduce")))
        return st;
    }
    return FA_OK;
  }
  a.dq_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.dq_off);
  if ((st = hip_status(fa::launch_zero_f32(a.dq_acc, (int64_t)p->B * p->Hq * p->Sq * p->D, stream), "dq clear")))
    return st;
  if ((st = hip_status(fa::launch_bwd(a, is_bf16, stream), "backward"))) return st;
  fa::DqArgs c;
  c.B = p->B;
  c.Hq = p->Hq;
  c.Sq = p->Sq;
  c.D = p->D;
  c.dq_acc = a.dq_acc;
  c.dq = dq->data;
  c.sdq = strides_of(dq);
  c.scale = p->scale;
  return hip_status(fa::launch_dq_convert(c, is_bf16, stream), "dq convert");
}

// Split of the bf16 forward's key walks: fwd_split when given, else 1 unless the grid has
// fewer than 256 query-tile workgroups (one per CU at most: a CU holds two), then as many
// as bring it near 512 while every split keeps at least 12 key tiles (capped at 16): the
// merge and each workgroup's first loads cost about as much as 12 tiles of walk
// (measured: 16 heads x 1542 rows gains 10% at 2 splits and loses at 3; a 512-row
// chunk over a 32768-key window runs 4x faster at 8).
int split_walk_shares(const fa_attn_params* p);

// Where the split walk would take two shares, a grid with no dense mask, ALiBi, causal diagonal
// or window (a key or query length at most) takes instead the forward variant whose workgroup
// splits its keys between its two wave pairs (64-row query tiles, the halves merged in LDS), with
// no merge pass: measured on MI355X, DiT self-attention with the pad given as a key length
// 37.4 -> 31.6 us; with a dense mask, under a band, for cross-attention and for causal chunks the
// split walk stayed faster.
bool fwd_key_halves(const fa_attn_params* p) {
  if (p->dtype != FA_BF16 || p->fwd_variant || p->fwd_split || p->mask || p->alibi || p->causal ||
      p->window_left >= 0 || p->window_right >= 0 || p->kv_format != FA_KV_DTYPE)
    return false;
  return split_walk_shares(p) == 2;
}

int choose_fwd_split(const fa_attn_params* p) {
  if (p->dtype != FA_BF16 || fwd_key_halves(p)) return 1;
  return split_walk_shares(p);
}

int split_walk_shares(const fa_attn_params* p) {
  const int64_t wgs = (int64_t)p->B * p->Hq * ((p->Sq + 127) / 128);
  int64_t nkt = (p->Sk + 63) / 64;
  if (p->causal) {  // the longest walk: the last query tile's
    const int64_t last_key = p->q_offset + p->Sq - 1;
    nkt = last_key < 0 ? 0 : std::min<int64_t>(last_key / 64 + 1, nkt);
  }
  if (p->window_left >= 0) {  // a band: a 128-row workgroup sees at most its rows' spans
    const int64_t right = p->window_right >= 0 ? p->window_right : (p->causal ? 0 : p->Sk);
    nkt = std::min<int64_t>(nkt, (p->window_left + right + 128) / 64 + 2);
  }
  if (p->fwd_split) return (int)std::max<int64_t>(1, std::min<int64_t>(p->fwd_split, std::max<int64_t>(nkt, 1)));
  if (wgs >= 256) return 1;
  const int64_t s = std::min<int64_t>({16, (512 + wgs - 1) / wgs, nkt / 12});
  return (int)std::max<int64_t>(1, s);
}

size_t fwd_workspace_bytes(const fa_attn_params* p) {
  const int s = choose_fwd_split(p);
  if (s <= 1) return 0;
  // bf16 rows (2 D bytes) plus their fp32 base and row sum (8 bytes)
  return round256((size_t)s * p->B * p->Hq * p->Sq * (2 * p->D + 8));
}

fa_status fwd_common(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                     const fa_view* o, const fa_view* lse, void* workspace, size_t workspace_bytes_given,
                     bool with_ws, hipStream_t stream) {
  fa_status s = check_params(p);
  if (s) return s;
  if (!with_ws && p->fwd_split > 1)
    return fail(FA_ERR_WORKSPACE, "fwd_split %d needs a workspace: call fa_train_fwd_ws", p->fwd_split);
  const int elt = elt_of(p);
  Extent eq, eo, el;
  Extent ins[6];
  const char* in_names[6] = {"q"};
  int n_in = 1;
  if ((s = check_view(q, "q", p->B, p->Hq, p->Sq, p->D, elt, true, false, &eq))) return s;
  ins[0] = eq;
  if ((s = check_kv(p, k, v, ins, &n_in, in_names))) return s;
  if ((s = check_view(o, "o", p->B, p->Hq, p->Sq, p->D, elt, true, true, &eo))) return s;
  if (!lse) return fail(FA_ERR_NULL, "lse view is NULL");
  if (lse->stride_s != 1) return fail(FA_ERR_STRIDE, "lse stride_s must be 1");
  if ((s = check_view(lse, "lse", p->B, p->Hq, p->Sq, 1, 4, false, true, &el))) return s;
  if (p->mask) {
    in_names[n_in] = "mask";
    ins[n_in++] = mask_extent(p);
  }
  const int splits = with_ws ? choose_fwd_split(p) : 1;
  const size_t need = splits > 1 ? fwd_workspace_bytes(p) : 0;
  if (need > 0) {
    if (!workspace) return fail(FA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes_given < need)
      return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_given, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(FA_ERR_ALIGN, "workspace is not 256-byte aligned");
  }
  const uintptr_t wlo = reinterpret_cast<uintptr_t>(workspace);
  Extent outs[3] = {eo, el, {wlo, wlo + need}};
  const char* out_names[3] = {"o", "lse", "workspace"};
  if ((s = check_alias(outs, need > 0 ? 3 : 2, out_names, ins, n_in, in_names))) return s;

#ifdef FA_CHECK
  if (p->dtype == FA_BF16) {  // the checked build verifies the launch's index space first
    char rep[256];
    Checker c{rep, sizeof rep};
    check_fwd(c, p, nullptr, nullptr);
    if (!c.ok) return fail(FA_ERR_HIP, "FA_CHECK: %s", rep);
  }
#endif
  fa::FwdArgs a;
  a.a = shape_of(p);
  a.q = q->data;
  a.k = k->data;
  a.v = v->data;
  a.o = o->data;
  a.lse = static_cast<float*>(lse->data);
  a.sq = strides_of(q);
  a.sk = strides_of(k);
  a.sv = strides_of(v);
  a.so = strides_of(o);
  a.lse_sb = lse->stride_b;
  a.lse_sh = lse->stride_h;
  a.inv_scale = 1.f / p->scale;
  const uintptr_t mp = reinterpret_cast<uintptr_t>(p->mask);
  a.mask_vec4 = p->mask && mp % 16 == 0 && p->mask_stride_q % 4 == 0 && p->mask_stride_b % 4 == 0 &&
                 p->mask_stride_h % 4 == 0;
  a.sinks = p->sinks;
  a.splits = splits;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (p->dtype == FA_BF16) {
    if (splits > 1) {  // the split walk runs the default configuration
      a.part_o = workspace;
      a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           (size_t)splits * p->B * p->Hq * p->Sq * p->D * 2);
      return hip_status(fa::launch_fwd_bf16_split(a, stream), "split forward");
    }
    // variant 1 (32 query rows per wave, 64-key tiles, two waves per SIMD) measured
    // faster than variant 2 (64 rows per wave, 32-key tiles, one wave per SIMD) on
    // every workload shape tried; variant 2 stays selectable for tuning
    const int variant = p->fwd_variant ? p->fwd_variant : (fwd_key_halves(p) ? 3 : 1);
    return hip_status(fa::launch_fwd_bf16(a, variant, stream), "forward");
  }
  return hip_status(fa::launch_fwd(a, 0, stream), "forward");
}


#ifdef FA_CHECK
// ---------------------------------------------------------------------------
// Checked build (-DFA_CHECK): the index space of every launch, verified on the host
// ---------------------------------------------------------------------------
// For a problem, the checker takes the library's own plan (split choices, workspace layout,
// unit counts) and enumerates every workgroup the bf16 forward and backward would launch,
// decoding each with the kernels' own unit decoding, row / key ranges and LDS offsets
// (shared host-device helpers), and verifies that every row it stages, every LDS offset it
// reads or writes, every row it stores and every workspace slice it touches lies inside its
// buffer, and that the units cover every output row exactly once (or once per split). The
// structured lengths are host copies here (the kernels read them on the device).
template <int D>
void check_tile_offsets(Checker& c, int rows, const char* what) {
  // every 16-byte chunk of a [rows][D] tile lands once inside the tile; transpose reads stay inside
  using TL = fa::Tile<D>;
  std::vector<int> seen((size_t)rows * D / 8, 0);
  for (int r = 0; r < rows; ++r)
    for (int ch = 0; ch < D / 8; ++ch) {
      const int off = TL::chunk(r, ch);
      if (off < 0 || off + 8 > rows * D || off % 8) return c.fail("%s: chunk (%d, %d) at %d", what, r, ch, off);
      if (seen[off / 8]++) return c.fail("%s: two chunks share LDS offset %d", what, off);
    }
  for (int r = 0; r < rows; ++r)
    for (int col = 0; col < D; col += 4) {
      const int off = TL::quad(r, col);
      if (off < 0 || off + 4 > rows * D) return c.fail("%s: transpose read (%d, %d) at %d", what, r, col, off);
    }
}

void check_bwd(Checker& c, const fa_attn_params* p, const int32_t* klen_h, const int32_t* qlen_h) {
  const fa::AttnShape a = shape_of(p);
  int kv, q, qt;
  choose_splits(p, false, &kv, &q, &qt);
  const int kv_role = p->softcap > 0.f || p->kv_format != FA_KV_DTYPE ? 0 : (p->bwd_kv_walk == 2 ? 1 : 0);
  fa::BwdPlan plan;
  const WsLayout wl = workspace_layout(p, false);
  fa::plan_bwd_bf16(a, kv, q, qt, 0, &plan, kv_role, wl.need_ds ? 1 : 0);
  const int64_t nq = (int64_t)p->B * p->Hq * p->Sq * p->D, nk = (int64_t)p->B * p->Hkv * p->Sk * p->D;
  if (wl.need_dq && (int64_t)(wl.dk_off - wl.dq_off) < plan.q_split * nq * 4) c.fail("dq slices exceed their space");
  if (wl.need_dkdv && (int64_t)(wl.dv_off - wl.dk_off) < plan.kv_split * nk * 4) c.fail("dk slices exceed their space");
  if (wl.need_dkdv && (int64_t)(wl.ds_off - wl.dv_off) < plan.kv_split * nk * 4) c.fail("dv slices exceed their space");
  if (wl.need_ds && wl.total - wl.ds_off < ds_bytes(p)) c.fail("stored dS exceeds its space");
  if (wl.need_ds && (plan.ds_nrt != (p->Sq + 63) / 64 || plan.ds_nku != (p->Sk + fa::kBwdUnit - 1) / fa::kBwdUnit))
    c.fail("stored dS block grid %d x %d", plan.ds_nrt, plan.ds_nku);
  const int KB = kv_role ? fa::kBwdRoleKeys : fa::kBwdUnit, BM = 64, G = p->Hq / p->Hkv;
  const int nkt = (p->Sk + KB - 1) / KB;
  if (plan.n_kv_units != nkt * p->B * p->Hkv * plan.kv_split) c.fail("dK/dV unit count %d", plan.n_kv_units);
  std::vector<int> kv_seen((size_t)nkt * p->B * p->Hkv * plan.kv_split, 0);
  for (int unit = 0; unit < plan.n_kv_units && c.ok; ++unit) {
    const fa::KvUnit u = fa::kv_unit_of(a, plan, unit);
    if (u.kt < 0 || u.kt >= nkt || u.b < 0 || u.b >= p->B || u.hk < 0 || u.hk >= p->Hkv || u.split < 0 ||
        u.split >= plan.kv_split)
      return c.fail("dK/dV unit %d decodes to (%d, %d, %d, %d)", unit, u.kt, u.b, u.hk, u.split);
    if (kv_seen[(((size_t)u.kt * p->B + u.b) * p->Hkv + u.hk) * plan.kv_split + u.split]++)
      return c.fail("dK/dV unit %d duplicates another", unit);
    const int klen = klen_h ? std::min(std::max(klen_h[u.b], 0), p->Sk) : p->Sk;
    const int qlen = qlen_h ? std::min(std::max(qlen_h[u.b], 0), p->Sq) : p->Sq;
    const int n0 = u.kt * KB;
    int qt0 = 0, qt_end = 0;
    if (n0 < klen) {
      int64_t lo, hi, lo1, hi1;
      fa::row_range(a, klen, qlen, n0, lo, hi);
      fa::row_range(a, klen, qlen, std::min(n0 + KB, klen) - 1, lo1, hi1);
      const int nqt = (p->Sq + BM - 1) / BM;
      qt0 = (int)std::min<int64_t>(lo / BM, nqt);
      qt_end = hi1 > lo ? (int)std::min<int64_t>((hi1 + BM - 1) / BM, nqt) : qt0;
      if (qt_end < qt0) qt_end = qt0;
    }
    const int npairs = (qt_end - qt0) * G;
    for (int pr = u.split; pr < npairs; pr += plan.kv_split) {
      const int h = u.hk * G + pr % G, q0 = (qt0 + pr / G) * BM;
      if (h >= p->Hq || q0 < 0 || q0 >= p->Sq) return c.fail("dK/dV unit %d walks pair (%d, %d)", unit, h, q0);
      // staged rows: the tile's buffer resource ends after row q0 + v - 1, v = min(BM, Sq - q0)
      // (later rows arrive as zeros)
      const int v = std::min(BM, p->Sq - q0);
      if (v < 1 || q0 + v - 1 >= p->Sq) return c.fail("dK/dV unit %d stages past Sq", unit);
      if (wl.need_ds) {  // the pair's stored dS block lies inside the workspace's dS region
        const int64_t blk = (((int64_t)u.b * p->Hq + h) * plan.ds_nku + u.kt) * plan.ds_nrt + q0 / BM;
        if (q0 / BM >= plan.ds_nrt || u.kt >= plan.ds_nku || (size_t)(blk + 1) * fa::kDsBlock > ds_bytes(p))
          return c.fail("dK/dV unit %d stores dS block %lld past its region", unit, (long long)blk);
      }
    }
    for (int w = 0; w < KB / 32; ++w) {
      const int kbase = n0 + 32 * w, rows = std::max(0, std::min(32, p->Sk - kbase));
      if (rows == 0) continue;  // a wave whose keys all lie past Sk stores nothing
      if (kbase + rows > p->Sk) return c.fail("dK/dV unit %d stores past Sk", unit);
      if (plan.kv_split > 1) {
        const int64_t end = (int64_t)u.split * nk + (((int64_t)u.b * p->Hkv + u.hk) * p->Sk + kbase + rows) * p->D;
        if (end > plan.kv_split * nk) return c.fail("dK/dV unit %d writes past its slices", unit);
      }
    }
  }
  for (size_t i = 0; i < kv_seen.size() && c.ok; ++i)
    if (kv_seen[i] != 1) c.fail("dK/dV unit %zu covered %d times", i, kv_seen[i]);
  // dQ units: each 128-row query tile of each head once, or once per split for the split tiles
  const int QM = plan.q_bm, QN = 64, nqt = (p->Sq + QM - 1) / QM;
  if (plan.n_q_units != (nqt - plan.q_tiles_split + plan.q_tiles_split * plan.q_split) * p->B * p->Hq)
    c.fail("dQ unit count %d", plan.n_q_units);
  std::vector<int> q_seen((size_t)nqt * p->B * p->Hq * std::max(1, plan.q_split), 0);
  for (int unit = 0; unit < plan.n_q_units && c.ok; ++unit) {
    const fa::QUnit u = fa::q_unit_of(a, plan, unit);
    if (u.qt < 0 || u.qt >= nqt || u.b < 0 || u.b >= p->B || u.h < 0 || u.h >= p->Hq || u.split < 0 ||
        u.split >= u.nsplit)
      return c.fail("dQ unit %d decodes to (%d, %d, %d, %d)", unit, u.qt, u.b, u.h, u.split);
    if (u.nsplit != (u.qt < plan.q_tiles_split ? plan.q_split : 1)) return c.fail("dQ unit %d: split count", unit);
    if (q_seen[(((size_t)u.qt * p->B + u.b) * p->Hq + u.h) * std::max(1, plan.q_split) + u.split]++)
      return c.fail("dQ unit %d duplicates another", unit);
    const int klen = klen_h ? std::min(std::max(klen_h[u.b], 0), p->Sk) : p->Sk;
    const int qlen = qlen_h ? std::min(std::max(qlen_h[u.b], 0), p->Sq) : p->Sq;
    const int q0 = u.qt * QM, nkt64 = (p->Sk + QN - 1) / QN;
    int kb = 0, ke = 0;
    if (q0 < qlen) {
      int64_t lo, hi, lo1, hi1;
      fa::key_range(a, klen, qlen, q0, lo, hi);
      fa::key_range(a, klen, qlen, std::min(q0 + QM, qlen) - 1, lo1, hi1);
      kb = (int)std::min<int64_t>(lo / QN, nkt64);
      ke = hi1 > lo ? (int)std::min<int64_t>((hi1 + QN - 1) / QN, nkt64) : kb;
      if (ke < kb) ke = kb;
    }
    for (int t = kb + u.split; t < ke; t += u.nsplit) {  // (a tile's resource ends at key min(t QN + QN, Sk) - 1)
      if (t * QN >= p->Sk) return c.fail("dQ unit %d walks key tile %d past Sk", unit, t);
      if (wl.need_ds)  // the half blocks it copies (row tiles past the last copy nothing)
        for (int w = 0; w < QM / 64; ++w) {
          const int rt = q0 / 64 + w;
          if (rt >= plan.ds_nrt) continue;
          const int64_t end = ((((int64_t)u.b * p->Hq + u.h) * plan.ds_nku + t / 2) * plan.ds_nrt + rt) * fa::kDsBlock +
                              (t % 2 + 1) * (fa::kDsBlock / 2);
          if (t / 2 >= plan.ds_nku || (size_t)end > ds_bytes(p))
            return c.fail("dQ unit %d reads dS past its region (tile %d)", unit, t);
        }
    }
    for (int w = 0; w < QM / 32; ++w) {
      const int qw = q0 + 32 * w, rows = std::max(0, std::min(32, p->Sq - qw));
      if (rows == 0) continue;  // a wave whose rows all lie past Sq stores nothing
      if (qw + rows > p->Sq) return c.fail("dQ unit %d stores past Sq", unit);
      if (u.nsplit > 1) {
        const int64_t end = (int64_t)u.split * nq + (((int64_t)u.b * p->Hq + u.h) * p->Sq + qw + rows) * p->D;
        if (end > plan.q_split * nq) return c.fail("dQ unit %d writes past its slices", unit);
      }
    }
  }
  for (int qi = 0; qi < nqt && c.ok; ++qi)
    for (int bh = 0; bh < p->B * p->Hq && c.ok; ++bh) {
      const int ns = qi < plan.q_tiles_split ? plan.q_split : 1;
      for (int sp = 0; sp < std::max(1, plan.q_split); ++sp) {
        const int n = q_seen[((size_t)qi * p->B * p->Hq + bh) * std::max(1, plan.q_split) + sp];
        if (n != (sp < ns ? 1 : 0)) return c.fail("dQ tile %d, head %d, split %d covered %d times", qi, bh, sp, n);
      }
    }
}

void check_fwd(Checker& c, const fa_attn_params* p, const int32_t* klen_h, const int32_t* qlen_h) {
  const fa::AttnShape a = shape_of(p);
  const int splits = choose_fwd_split(p);
  const size_t need = splits > 1 ? fwd_workspace_bytes(p) : 0;
  const int64_t rows = (int64_t)p->B * p->Hq * p->Sq;
  if (splits > 1 && (size_t)(splits * rows * (2 * p->D + 8)) > need) c.fail("forward partials exceed the workspace");
  const int BM = 128, BN = 64, nkt = (p->Sk + BN - 1) / BN, nqt = (p->Sq + BM - 1) / BM;
  for (int b = 0; b < p->B && c.ok; ++b)
    for (int qi = 0; qi < nqt && c.ok; ++qi) {
      const int klen = klen_h ? std::min(std::max(klen_h[b], 0), p->Sk) : p->Sk;
      const int qlen = qlen_h ? std::min(std::max(qlen_h[b], 0), p->Sq) : p->Sq;
      const int q0 = qi * BM;
      int kb = 0, ke = 0;
      if (q0 < qlen) {
        int64_t lo, hi, lo1, hi1;
        fa::key_range(a, klen, qlen, q0, lo, hi);
        fa::key_range(a, klen, qlen, std::min(q0 + BM, qlen) - 1, lo1, hi1);
        kb = (int)std::min<int64_t>(lo / BN, nkt);
        ke = hi1 > lo ? (int)std::min<int64_t>((hi1 + BN - 1) / BN, nkt) : 0;
        if (ke < kb) ke = kb;
      }
      for (int z = 0; z < splits; ++z) {  // the z-th share of [kb, ke)
        const int per = (ke - kb + splits - 1) / splits;
        const int b0 = std::min(ke, kb + z * per), e0 = std::min(ke, b0 + per);
        for (int t = b0; t < e0; ++t)
          if (t * BN >= p->Sk) return c.fail("forward tile (%d, %d) walks key tile %d past Sk", b, qi, t);
      }
      for (int w = 0; w < 4; ++w) {
        const int row = q0 + 32 * w + 31;  // the last row a wave may store (rows past Sq are skipped)
        if (splits > 1 && std::min(row, p->Sq - 1) >= p->Sq) return c.fail("forward stores past Sq");
      }
    }
}

#endif  // FA_CHECK
}  // namespace

extern "C" {

fa_status fa_train_fwd(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                       const fa_view* o, const fa_view* lse, hipStream_t stream) {
  g_err[0] = 0;
  return fwd_common(p, q, k, v, o, lse, nullptr, 0, false, stream);
}

size_t fa_train_fwd_workspace_bytes(const fa_attn_params* p) {
  if (check_params(p) != FA_OK) return (size_t)-1;
  return fwd_workspace_bytes(p);
}

fa_status fa_train_fwd_ws(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                          const fa_view* o, const fa_view* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  g_err[0] = 0;
  return fwd_common(p, q, k, v, o, lse, workspace, workspace_bytes, true, stream);
}

fa_status fa_train_bwd_preprocess(const fa_attn_params* p, const fa_view* o, const fa_view* dout,
                                  const fa_view* delta, hipStream_t stream) {
  g_err[0] = 0;
  if (!p) return fail(FA_ERR_NULL, "params pointer is NULL");
  if (p->B < 1 || p->Hq < 1 || p->Sq < 1) return fail(FA_ERR_SHAPE, "sizes must be positive");
  if (p->dtype != FA_F32 && p->dtype != FA_BF16) return fail(FA_ERR_DTYPE, "unknown dtype %d", p->dtype);
  if (p->D != 64 && p->D != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", p->D);
  const int elt = elt_of(p);
  Extent eo, edo, ed;
  fa_status s;
  if ((s = check_view(o, "o", p->B, p->Hq, p->Sq, p->D, elt, true, false, &eo))) return s;
  if ((s = check_view(dout, "dout", p->B, p->Hq, p->Sq, p->D, elt, true, false, &edo))) return s;
  if (!delta) return fail(FA_ERR_NULL, "delta view is NULL");
  if (delta->stride_s != 1) return fail(FA_ERR_STRIDE, "delta stride_s must be 1");
  if ((s = check_view(delta, "delta", p->B, p->Hq, p->Sq, 1, 4, false, true, &ed))) return s;
  Extent ins[2] = {eo, edo};
  const char* in_names[2] = {"o", "dout"};
  const char* out_names[1] = {"delta"};
  if ((s = check_alias(&ed, 1, out_names, ins, 2, in_names))) return s;
  fa::PreArgs a;
  a.B = p->B;
  a.Hq = p->Hq;
  a.Sq = p->Sq;
  a.D = p->D;
  a.o = o->data;
  a.dout = dout->data;
  a.delta = static_cast<float*>(delta->data);
  a.so = strides_of(o);
  a.sdo = strides_of(dout);
  a.delta_sb = delta->stride_b;
  a.delta_sh = delta->stride_h;
  return hip_status(fa::launch_preprocess(a, p->dtype == FA_BF16, stream), "preprocess");
}

fa_status fa_train_bwd_sinks(const fa_attn_params* p, const fa_view* lse, const fa_view* delta, float* dsink,
                             hipStream_t stream) {
  g_err[0] = 0;
  fa_status s = check_params(p);
  if (s) return s;
  if (!p->sinks) return fail(FA_ERR_NULL, "the params carry no sinks");
  if (!dsink) return fail(FA_ERR_NULL, "dsink is NULL");
  if (reinterpret_cast<uintptr_t>(dsink) % 4) return fail(FA_ERR_ALIGN, "dsink is not 4-byte aligned");
  Extent el, ed;
  for (const fa_view* v : {lse, delta}) {
    if (!v) return fail(FA_ERR_NULL, "lse / delta view is NULL");
    if (v->stride_s != 1) return fail(FA_ERR_STRIDE, "lse / delta stride_s must be 1");
  }
  if ((s = check_view(lse, "lse", p->B, p->Hq, p->Sq, 1, 4, false, false, &el))) return s;
  if ((s = check_view(delta, "delta", p->B, p->Hq, p->Sq, 1, 4, false, false, &ed))) return s;
  const uintptr_t d0 = reinterpret_cast<uintptr_t>(dsink), s0 = reinterpret_cast<uintptr_t>(p->sinks);
  const Extent eds = {d0, d0 + (uintptr_t)p->Hq * 4}, es = {s0, s0 + (uintptr_t)p->Hq * 4};
  if (overlaps(eds, el) || overlaps(eds, ed) || overlaps(eds, es))
    return fail(FA_ERR_ALIAS, "dsink overlaps the LSE, Delta or the sinks");
  fa::SinkArgs a;
  a.B = p->B;
  a.Hq = p->Hq;
  a.Sq = p->Sq;
  a.sinks = p->sinks;
  a.lse = static_cast<const float*>(lse->data);
  a.delta = static_cast<const float*>(delta->data);
  a.lse_sb = lse->stride_b;
  a.lse_sh = lse->stride_h;
  a.delta_sb = delta->stride_b;
  a.delta_sh = delta->stride_h;
  a.dsink = dsink;
  return hip_status(fa::launch_sink_grad(a, stream), "sink gradient");
}

fa_status fa_train_dequant_q8_0(int32_t B, int32_t H, int32_t S, int32_t D, const fa_view* qs, const fa_view* d,
                                const fa_view* out, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 1 || H < 1 || S < 1) return fail(FA_ERR_SHAPE, "B, H and S must be positive");
  if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", D);
  Extent eq, ed, eo;
  fa_status s;
  if ((s = check_view(qs, "qs", B, H, S, D, 1, true, false, &eq))) return s;
  if ((s = check_view(d, "d", B, H, S, D / 32, 2, false, false, &ed))) return s;
  if ((s = check_view(out, "out", B, H, S, D, 2, true, true, &eo))) return s;
  if (d->stride_s < D / 32 && S > 1) return fail(FA_ERR_STRIDE, "d: stride_s must cover the row's D / 32 scales");
  if (overlaps(eo, eq) || overlaps(eo, ed)) return fail(FA_ERR_ALIAS, "out overlaps qs or d");
  fa::DequantArgs a;
  a.B = B;
  a.H = H;
  a.S = S;
  a.D = D;
  a.qs = static_cast<const int8_t*>(qs->data);
  a.d = static_cast<const _Float16*>(d->data);
  a.out = out->data;
  a.sq = strides_of(qs);
  a.sd = strides_of(d);
  a.so = strides_of(out);
  return hip_status(fa::launch_dequant_q8_0(a, stream), "q8_0 dequant");
}

fa_status fa_train_convert_f16(int32_t B, int32_t H, int32_t S, int32_t D, const fa_view* src, const fa_view* out,
                               int32_t out_dtype, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 1 || H < 1 || S < 1) return fail(FA_ERR_SHAPE, "B, H and S must be positive");
  if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", D);
  if (out_dtype != FA_F32 && out_dtype != FA_BF16) return fail(FA_ERR_DTYPE, "unknown out dtype %d", out_dtype);
  Extent es, eo;
  fa_status s;
  if ((s = check_view(src, "src", B, H, S, D, 2, true, false, &es))) return s;
  if ((s = check_view(out, "out", B, H, S, D, out_dtype == FA_F32 ? 4 : 2, true, true, &eo))) return s;
  if (overlaps(eo, es)) return fail(FA_ERR_ALIAS, "out overlaps src");
  fa::ConvertArgs a;
  a.B = B;
  a.H = H;
  a.S = S;
  a.D = D;
  a.src = static_cast<const _Float16*>(src->data);
  a.out = out->data;
  a.to_bf16 = out_dtype == FA_BF16;
  a.ss = strides_of(src);
  a.so = strides_of(out);
  return hip_status(fa::launch_convert_f16(a, stream), "f16 conversion");
}

size_t fa_train_bwd_workspace_bytes(const fa_attn_params* p) {
  if (check_params(p) != FA_OK) return (size_t)-1;
  return workspace_bytes(p);
}

fa_status fa_train_bwd(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                       const fa_view* dout, const fa_view* lse, const fa_view* delta, const fa_view* dq,
                       const fa_view* dk, const fa_view* dv, void* workspace, size_t workspace_bytes_given,
                       hipStream_t stream) {
  g_err[0] = 0;
  return bwd_common(p, q, k, v, dout, lse, delta, dq, dk, dv, workspace, workspace_bytes_given, stream, false);
}

fa_status fa_train_bwd_noalloc(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                               const fa_view* dout, const fa_view* lse, const fa_view* delta, const fa_view* dq,
                               const fa_view* dk, const fa_view* dv, hipStream_t stream) {
  g_err[0] = 0;
  return bwd_common(p, q, k, v, dout, lse, delta, dq, dk, dv, nullptr, 0, stream, false, true);
}

fa_status fa_train_bwd_chunked(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                               const fa_view* dout, const fa_view* lse, const fa_view* delta, const fa_view* dq,
                               const fa_view* dk_acc, const fa_view* dv_acc, void* workspace,
                               size_t workspace_bytes_given, hipStream_t stream) {
  g_err[0] = 0;
  return bwd_common(p, q, k, v, dout, lse, delta, dq, dk_acc, dv_acc, workspace, workspace_bytes_given, stream,
                    true);
}

size_t fa_train_mask_tiles_bytes(const fa_attn_params* p) {
  if (check_params(p) != FA_OK || !p->mask) return 0;
  const int64_t nblk = tile_batches(p) * tile_rows(p) * tile_cols(p);
  return (size_t)((nblk + 255) / 256 * 256 + 2 * nblk * 64 * 8);  // classes, row words, column words
}

fa_status fa_train_mask_tiles(const fa_attn_params* p, uint8_t* tiles, hipStream_t stream) {
  g_err[0] = 0;
  fa_status s = check_params(p);
  if (s) return s;
  if (!p->mask) return fail(FA_ERR_NULL, "the params carry no mask");
  if (p->mask_stride_h > 0) return fail(FA_ERR_UNSUPPORTED, "the mask block map is per batch entry, not per head");
  if (!tiles) return fail(FA_ERR_NULL, "tiles is NULL");
  const uintptr_t t = reinterpret_cast<uintptr_t>(tiles);
  if (t % 8) return fail(FA_ERR_ALIGN, "tiles is not 8-byte aligned");
  const Extent et = {t, t + (uintptr_t)fa_train_mask_tiles_bytes(p)};
  const Extent em = mask_extent(p);
  if (overlaps(et, em)) return fail(FA_ERR_ALIAS, "tiles overlaps the mask");
  fa_attn_params q = *p;
  q.mask_tiles = tiles;
  return hip_status(fa::launch_mask_tiles(shape_of(&q), tiles, stream), "mask tiles");
}

const char* fa_train_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer";
    case FA_ERR_SHAPE: return "bad shape";
    case FA_ERR_DTYPE: return "bad dtype";
    case FA_ERR_STRIDE: return "bad stride";
    case FA_ERR_ALIGN: return "misaligned pointer or stride";
    case FA_ERR_ALIAS: return "output aliases another buffer";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

const char* fa_train_last_error(void) { return g_err; }

#ifdef FA_CHECK
// Checked build only: runs the host checker over the bf16 forward's and backward's launches for
// p (lengths as host arrays, or NULL for the full lengths). Returns FA_OK, or FA_ERR_HIP with
// the first violation in `report`.
fa_status fa_train_check_launch(const fa_attn_params* p, const int32_t* key_len_host, const int32_t* q_len_host,
                                char* report, size_t report_len) {
  g_err[0] = 0;
  fa_status s = check_params(p);
  if (s) return s;
  if (p->dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "the checker covers the bf16 kernels");
  Checker c{report, report_len};
  if (report_len) report[0] = 0;
  check_tile_offsets<64>(c, 64, "tile D=64");
  check_tile_offsets<128>(c, 64, "tile D=128");
  check_fwd(c, p, key_len_host, q_len_host);
  if (!generic_path(p)) check_bwd(c, p, key_len_host, q_len_host);  // (the generic kernels have no plan)
  return c.ok ? FA_OK : fail(FA_ERR_HIP, "FA_CHECK: %s", report);
}
#endif

int fa_train_version(void) { return FA_TRAIN_ABI_VERSION; }

}  // extern "C"
