/*
 * fa_train.h -- C ABI of the fused flash-attention training op for MI355X (gfx950).
 *
 * The op is exact softmax attention with a per-row log-sum-exp (LSE) side output,
 * and its gradient, split the way the pages split it:
 *
 *   fa_train_fwd             O and LSE                         (forward)
 *   fa_train_bwd_preprocess  Delta_i = sum_d dO_id * O_id      (the step between the
 *                            forward's LSE and the gradients)
 *   fa_train_bwd             dQ, dK, dV from Q, K, V, dO, LSE, Delta
 *   fa_train_bwd_chunked     the same, but dK/dV are ADDED into caller-owned fp32
 *                            accumulators over a cached K/V window (exact walk)
 *
 * Definitions (natural log; s = scale; G = Hq / Hkv; query head h reads KV head h / G):
 *   S_ij  = s * <q_i, k_j> + M_ij, or -inf when masked (mask entry -inf, causal
 *           j > q_offset + i)
 *   LSE_i = ln sum_j exp(S_ij);  P_ij = exp(S_ij - LSE_i);  O_i = sum_j P_ij v_j
 *   a query row with no visible key is "fully masked": O_i = 0 and LSE_i = 0
 *   dS_ij = P_ij (<dO_i, v_j> - Delta_i);  dQ_i = s sum_j dS_ij k_j
 *   dK_j  = s sum_{h in group} sum_i dS_ij q_i;  dV_j = sum_{h in group} sum_i P_ij dO_i
 *
 * Sources: "Flash Attn Training" skill page, section 6 (trap 3: the forward emits
 * O and the LSE and the LSE receives no gradient; trap 4: the backward refuses to
 * write over the forward's buffers; trap 5: native GQA without head expansion;
 * traps 8 and 9: fully masked rows give O = 0, LSE = 0 and fully masked key columns
 * get zero gradient); llama.cpp pull request 57, commit 86c140d (the backward runs
 * over KV-window tiles, first the per-row LSE, then Delta, then the gradients of each
 * tile, and adds each query group's dK/dV into its one KV head; the exact walk adds
 * the gradient of the cached K/V into an accumulator that the caller owns) and the commit that makes
 * the training graph the serving graph (attention reads the cache in place).
 *
 * Conventions shared by every entry point
 *   - Device pointers throughout. Q, O, dO, dQ are [B, Hq, Sq, D]; K, V, dK, dV are
 *     [B, Hkv, Sk, D]; each is described by an fa_view: element strides for the
 *     batch, head and sequence dimensions, with D contiguous. LSE and Delta are fp32
 *     [B, Hq, Sq] views whose sequence stride must be 1.
 *   - dtype applies to Q, K, V, O, dO, dQ, dK, dV. Accumulation is fp32 for both
 *     dtypes; with FA_BF16 the probabilities and dS are rounded to bf16 before
 *     their matrix products.
 *   - Rows need 16-byte alignment: data pointers 16-byte aligned and every stride a
 *     multiple of 16 bytes' worth of elements; stride_s must be below 2^24 elements.
 *   - The mask is optional, fp32, additive, indexed [b][i][j] (j contiguous), with
 *     values 0, finite biases or -inf. mask_stride_b = 0 shares one mask across the
 *     batch. It is broadcast over heads.
 *   - Work is enqueued on `stream` (NULL = the null stream). The library never
 *     allocates, frees, synchronizes or reads results back; outputs are valid once
 *     the stream's work has completed. Entry points are reentrant.
 *   - Every argument check runs on the host before any launch; on error nothing is
 *     launched, outputs are untouched, and fa_train_last_error() describes the
 *     problem (thread-local text).
 */
#ifndef FA_TRAIN_H
#define FA_TRAIN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_TRAIN_ABI_VERSION 14

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,       /* non-positive size, Hq % Hkv != 0, bad q_offset, ... */
    FA_ERR_DTYPE = 3,       /* unknown dtype */
    FA_ERR_STRIDE = 4,      /* stride too small / overlapping rows, LSE stride_s != 1 */
    FA_ERR_ALIGN = 5,       /* pointer or stride not 16-byte aligned */
    FA_ERR_ALIAS = 6,       /* an output overlaps an input or another output */
    FA_ERR_UNSUPPORTED = 7, /* head dim other than 64 or 128 */
    FA_ERR_WORKSPACE = 8,   /* workspace missing or smaller than fa_train_bwd_workspace_bytes */
    FA_ERR_HIP = 9          /* a kernel launch failed; detail in fa_train_last_error() */
} fa_status;

typedef enum fa_dtype { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/* A strided view of a [B, H, S, D] tensor (or [B, H, S] for LSE / Delta).
 * Strides count elements of the view's own type. D is contiguous. */
typedef struct fa_view {
    void* data;
    int64_t stride_b;
    int64_t stride_h;
    int64_t stride_s;
} fa_view;

typedef struct fa_attn_params {
    int32_t B, Hq, Hkv, Sq, Sk, D;
    int32_t dtype;        /* fa_dtype */
    int32_t causal;       /* 0 or 1: key j visible to query i only if j <= q_offset + i */
    int64_t q_offset;     /* key position of query row 0 (Sk - Sq for bottom-right causal; rows with
                             q_offset + i < 0 see no key under causal masking) */
    float scale;          /* multiplies <q, k>; must be > 0; usually 1/sqrt(D) */
    const float* mask;    /* optional additive mask [b][i][j], fp32; NULL = none */
    int64_t mask_stride_b;/* elements between batch entries; 0 = shared by the batch */
    int64_t mask_stride_q;/* elements between query rows (>= Sk) */
    const uint8_t* mask_tiles; /* optional classification of the mask's 64 x 64 blocks made by
                             fa_train_mask_tiles for this very mask (same pointer, strides and
                             shape); NULL = every block is read elementwise. With it, blocks
                             that are entirely -inf are skipped and blocks that are entirely
                             0 are not read. */
    /* Work decomposition hints, 0 = automatic (the normal setting; other values are
     * for tuning and give the same results up to fp32 summation order): */
    int32_t fwd_variant;  /* bf16 forward: 1 = 32 query rows per wave, 64-key tiles;
                             2 = 64 rows per wave, 32-key tiles; 3 = keys split over two
                             halves of the workgroup, merged at the end */
    int32_t kv_split;     /* bf16 backward: workgroups sharing one 128-key tile's dK/dV
                             walk, 1 .. 64 (> 1: each writes an fp32 partial slice in the
                             workspace, summed by a reduce pass) */
    int32_t q_split;      /* bf16 backward: workgroups sharing one split 128-row query tile's
                             dQ walk, 1 .. 64 (> 1: fp32 partial slices, as for kv_split);
                             which tiles are split: q_split_tiles below */
    int32_t fwd_split;    /* bf16 forward through fa_train_fwd_ws: workgroups sharing one
                             128-row query tile's key walk, 1 .. 64 (> 1: each stores its
                             rows normalised by its own row sum, in bf16, with their fp32
                             exponent base and row sum, in the workspace, and a merge pass
                             combines them). fa_train_fwd never splits and rejects > 1. */
    /* Structured masks (both dtypes; they combine with causal and with a dense mask): the
     * per-element padding and sliding-window masks of the pages' DiT batches ("sa" =
     * sliding window + padded key columns, "sa_pad" = padded key columns) without a
     * dense tensor. Entry (b, i, j) is hidden when j >= key_len[b], when i >= q_len[b]
     * (the row is then fully masked: O = 0, LSE = 0, dQ = 0, and it adds nothing to dK,
     * dV), when j < q_offset + i - window_left, or when j > q_offset + i + window_right. */
    const int32_t* key_len;  /* device [B] int32, each in [0, Sk] (clamped); NULL = Sk */
    const int32_t* q_len;    /* device [B] int32, each in [0, Sq] (clamped); NULL = Sq */
    int32_t window_left;     /* >= 0: keys at most this far before a row's position q_offset + i;
                                -1: no bound */
    int32_t window_right;    /* >= 0: keys at most this far after it; -1: no bound */
    /* Work decomposition hint of the bf16 backward, like the split hints above (same
     * results up to fp32 summation order): 0 = automatic (3 when the dQ grid has at least
     * 512 128-row tiles and the stored dS fits 2 GB, except in fa_train_bwd_noalloc; otherwise
     * 1 or 2), 1 = the dQ
     * workgroups share the dK/dV workgroups' launch, 2 = they run as a second kernel after
     * it, two per compute unit (chosen automatically for grids of at least 512 dQ
     * workgroups when dS is not stored), 3 = dQ from
     * stored dS: the dK/dV walk also writes every dS = P (dP - Delta) it forms (bf16, as its
     * dK product takes it) into the workspace, and a second kernel forms dQ = scale dS K
     * from it instead of recomputing S and dP (fewer matrix products, 2 bytes of traffic
     * each way per visible score; dK and dV are bitwise those of the other settings, dQ
     * differs only by the rounding of dS). The workspace then holds 16 KB per (batch entry,
     * query head, 64-row query tile, 128-key tile). Value 3 is taken as 0 with a stored
     * K/V window (kv_format), a mask gradient (dbias) or bwd_kv_walk = 2. 4 = as 2, with the
     * dQ kernel on a second stream of the library's (one per device, default priority),
     * forked from and joined back to the caller's stream by events, so that it runs beside
     * the dK/dV kernel on the compute units that one leaves free (the call stays ordered on the
     * caller's stream, and HIP graph capture records the fork and join); in
     * fa_train_bwd_noalloc it is taken as 2. */
    int32_t bwd_dq_launch;
    /* Attention sinks (both dtypes): one more logit per query head that joins every row's
     * softmax denominator and has no value row (llama.cpp pull request 57 lists sinks
     * among the score modifiers its flash backward lacked). sinks[h] is a natural-log
     * logit, used as given (not scaled): LSE_i = ln(sum_j exp(S_ij) + exp(sinks[h])), and
     * O_i = sum_j exp(S_ij - LSE_i) v_j. A row whose every key is masked then has
     * O = 0 and LSE = sinks[h]. The backward is unchanged (it reads the LSE); the sinks'
     * own gradient comes from fa_train_bwd_sinks. */
    const float* sinks;      /* device [Hq] fp32, 4-byte aligned; NULL = none */
    /* ALiBi (both dtypes; combines with every mask): a per-head linear penalty on the distance
     * between a key and the query's position, one of the score modifiers the pull request's
     * flash backward lacked. Score (b, h, i, j) gets -alibi[h] * |j - (q_offset + i)|, added
     * like a mask value (after the scale); under a causal mask that is the usual
     * alibi[h] * (j - q_offset - i). Positions are exact while |j - q_offset - i| < 2^24. It
     * is a constant of the scores, so the backward's gradients need nothing more. */
    const float* alibi;      /* device [Hq] fp32 slopes, 4-byte aligned; NULL = none */
    /* Work decomposition hint of the bf16 backward (same results up to fp32 summation
     * order): how many 128-row query tiles, counted from the first (their dQ workgroups
     * are dispatched last), have their dQ walk split q_split ways; the other tiles walk
     * whole. 0 = all tiles when q_split is given, else automatic. Splitting only the last
     * units to run shortens the end of the launch, when few compute units are busy. */
    int32_t q_split_tiles;
    /* Head stride of the mask, in elements: 0 = one mask for every head (the layout above);
     * > 0 = a mask per query head, entry (b, h, i, j) at mask + b * mask_stride_b +
     * h * mask_stride_h + i * mask_stride_q + j -- an additive score bias per head (the
     * pull request's KQ bias), with -inf still hiding entries; its gradient comes out through
     * dbias below. A per-head mask takes no mask block map (mask_tiles must be NULL). */
    int64_t mask_stride_h;
    /* Logit softcap (0 = none; else > 0 and finite), a score modifier the pull request's flash
     * backward lacked: score (b, h, i, j) = c * tanh(scale * <q_i, k_j> / c) + the mask value,
     * so the product is bounded by c before the mask and ALiBi are added; the backward
     * carries 1 - tanh^2 into dS. The bf16 kernels apply it in their MFMA walks (every work
     * decomposition); fp32 runs on the generic kernels. It combines with every mask (dense,
     * per head, structured), with sinks and with ALiBi. */
    float softcap;
    /* Work decomposition hint of the bf16 backward's dK/dV walk (same results up to fp32
     * summation order and one bf16 rounding of P inside dS): 0 = automatic (walk 1); 1 = one
     * wave per 32 keys computes S, dP, dV and dK (128-key workgroups, one per compute unit);
     * 2 = the work split by role, one wave computing S, P and dV and another dP, dS and dK for
     * each 32 keys (64-key workgroups, two per compute unit, P passed between them in bf16;
     * the dQ walk then runs as its own kernel). A logit softcap always takes walk 1. */
    int32_t bwd_kv_walk;
    /* Storage of K and V (bf16 problems only): FA_KV_DTYPE = the dtype above; FA_KV_F16 = fp16
     * values; FA_KV_Q8_0 = ggml's q8_0 blocks held as two planes, int8 quants in the k / v views
     * (element = byte strides) and one fp16 scale per 32 consecutive values along D in
     * k_scale / v_scale ([B, Hkv, Sk, D / 32], element strides), the stored value being
     * scale * quant. The kernels convert every K / V value they read to bf16 (fp16 widened
     * exactly, the q8_0 product exact in fp32, then one rounding to nearest even), so a
     * quantised or fp16 K/V window is attended to and trained in place, with no bf16 copy
     * (llama.cpp pull request 57: a q8_0 cache trains in place). dK and dV are the gradients
     * of the stored values, in the output dtype (bf16) or added into fp32 accumulators by
     * fa_train_bwd_chunked. Not combined with a dense mask, ALiBi or a logit softcap
     * (FA_ERR_UNSUPPORTED). */
    int32_t kv_format;
    fa_view k_scale;
    fa_view v_scale;
    /* The gradient of the additive mask, for a learnable score bias (the pull request's KQ
     * bias): an optional fp32 output of the backward entry points (fa_train_bwd,
     * fa_train_bwd_chunked, fa_train_bwd_noalloc). For every score it adds
     * dL/dM_ij = P_ij (dP_ij - Delta_i) (0 where the entry is hidden) into
     * dbias + b * dbias_stride_b + h * dbias_stride_h + i * dbias_stride_q + j: the caller
     * zeroes it before the first call, and the chunked walk's chunks sum into it. Its broadcast
     * follows the mask's: dbias_stride_b is 0 exactly when mask_stride_b is 0 (the batch
     * entries then add into one plane), dbias_stride_h is 0 exactly when mask_stride_h is 0
     * (the heads add into one plane); dbias_stride_q >= Sk; rows must not overlap. Needs a
     * dense mask (FA_ERR_SHAPE without one); a bf16 problem with a logit softcap does not take
     * it (FA_ERR_UNSUPPORTED). NULL: not computed. */
    float* dbias;
    int64_t dbias_stride_b, dbias_stride_h, dbias_stride_q;
} fa_attn_params;

#define FA_KV_DTYPE 0
#define FA_KV_F16 1
#define FA_KV_Q8_0 2

/* Forward: writes O (dtype) and LSE (fp32, natural log). Fully masked rows get
 * O = 0 and LSE = 0. O must not overlap Q, K or V. */
fa_status fa_train_fwd(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                       const fa_view* o, const fa_view* lse, hipStream_t stream);

/* Bytes of device workspace fa_train_fwd_ws needs for p: 0 when the forward is not
 * split, else splits * B * Hq * Sq * (2 D + 8) rounded up to 256 (each share's rows
 * normalised by its own row sum, in bf16, then their fp32 exponent bases and row sums). The split is fwd_split when set, else chosen
 * from the shape: only grids with fewer than 256 query-tile workgroups and key walks of
 * at least 24 tiles of 64 keys are split. Returns (size_t)-1 if p is invalid. */
size_t fa_train_fwd_workspace_bytes(const fa_attn_params* p);

/* Forward with a caller-owned workspace: the results of fa_train_fwd (O, LSE, fully
 * masked rows O = 0 and LSE = 0) for the same inputs, but a short grid may split each
 * query tile's key walk over several workgroups (the split-key reading of the pages'
 * tiled forward). Each share stores its rows normalised by its own row sum, rounded to
 * bf16, and the merge weights them by their row sums rescaled to the largest exponent
 * base: the LSE matches up to fp32 summation order, O up to one more bf16 rounding of
 * each share's row. `workspace`: at least
 * fa_train_fwd_workspace_bytes(p) bytes of device memory, 256-byte aligned (NULL
 * allowed when 0 bytes are needed), overlapping no input or output; contents on entry
 * do not matter. Errors: those of fa_train_fwd, FA_ERR_WORKSPACE, FA_ERR_ALIGN and
 * FA_ERR_ALIAS for the workspace. */
fa_status fa_train_fwd_ws(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                          const fa_view* o, const fa_view* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Preprocess for the backward: Delta_i = sum_d dO_id * O_id in fp32, from the stored
 * O and dO. Only B, Hq, Sq, D and dtype of p are used. */
fa_status fa_train_bwd_preprocess(const fa_attn_params* p, const fa_view* o, const fa_view* dout,
                                  const fa_view* delta, hipStream_t stream);

/* Bytes of device workspace fa_train_bwd / fa_train_bwd_chunked need for p (fp32
 * accumulators for split work, the stored dS with bwd_dq_launch = 3; may be 0). Returns
 * (size_t)-1 if p is invalid. */
size_t fa_train_bwd_workspace_bytes(const fa_attn_params* p);

/* Backward: OVERWRITES dQ, dK, dV (dtype). Reads Q, K, V, dO, the forward's LSE and
 * the preprocess's Delta. dQ/dK/dV must not overlap any input or each other (in
 * particular not the forward's O / LSE buffers). `workspace` is caller-owned device
 * memory of at least fa_train_bwd_workspace_bytes(p) bytes, 256-byte aligned; its
 * contents on entry do not matter. dK/dV rows of keys no query can see are zero. */
fa_status fa_train_bwd(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                       const fa_view* dout, const fa_view* lse, const fa_view* delta, const fa_view* dq,
                       const fa_view* dk, const fa_view* dv, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Chunked backward for the exact walk over a cached K/V window: the query chunk
 * (Sq rows at key positions q_offset ...) attends to window rows [0, Sk). OVERWRITES
 * dQ for the chunk and ADDS the chunk's dK/dV contributions into fp32 accumulators
 * dk_acc / dv_acc, views over the window ([B, Hkv, >= Sk, D], fp32 element strides).
 * The accumulators are never cleared by the library; the caller zeroes them before
 * the first chunk. Chunks may run in any order (the result is a sum). */
fa_status fa_train_bwd_chunked(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                               const fa_view* dout, const fa_view* lse, const fa_view* delta,
                               const fa_view* dq, const fa_view* dk_acc, const fa_view* dv_acc,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the static scratch array behind fa_train_bwd_noalloc (64 MiB per device). */
#define FA_TRAIN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* fa_train_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight training loops, harnesses that forbid allocation): the same
 * arguments, checks and results, but no workspace argument. The backward's workspace
 * (see fa_train_bwd_workspace_bytes: the split walks' fp32 slices, or the fp32 path's
 * dQ accumulator, which it clears itself with a kernel) is taken from a static device
 * array of FA_TRAIN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device
 * it runs on until the process ends; its device address is looked up on the first
 * call on each device, with that device current. Nothing is allocated or freed, by
 * the library or by any library it calls. A problem whose workspace would exceed the
 * array is rejected with FA_ERR_WORKSPACE before anything is launched (a smaller
 * kv_split / q_split hint, or fa_train_bwd with a caller-owned workspace, serves it).
 * Every call on one device shares that device's array and the array keeps the last
 * call's contents, so calls that may overlap on one device (on different streams, or
 * from different host threads without ordering) race: order them on one stream. */
fa_status fa_train_bwd_noalloc(const fa_attn_params* p, const fa_view* q, const fa_view* k, const fa_view* v,
                               const fa_view* dout, const fa_view* lse, const fa_view* delta, const fa_view* dq,
                               const fa_view* dk, const fa_view* dv, hipStream_t stream);

/* Mask block classes written by fa_train_mask_tiles. */
#define FA_TILE_DEAD 0  /* every entry of the block is -inf */
#define FA_TILE_OPEN 1  /* every entry of the block is exactly 0 */
#define FA_TILE_BITS 2  /* entries are 0 or -inf, both present: a visibility pattern */
#define FA_TILE_BIAS 3  /* some entry is a finite non-zero bias */
#define FA_MASK_TILE 64 /* block edge, in query rows and keys */

/* Bytes of the mask tile map for p (0 if p has no mask or is invalid). With
 * nblk = Bm * ceil(Sq/64) * ceil(Sk/64) (Bm = 1 when mask_stride_b == 0, else B), the
 * map starts with nblk class bytes, block (bm, rt, ct) at (bm * ceil(Sq/64) + rt) *
 * ceil(Sk/64) + ct, followed by per-block visibility bit words for the kernels. */
size_t fa_train_mask_tiles_bytes(const fa_attn_params* p);

/* Classifies every 64 x 64 block of p's mask (clipped at Sq and Sk) into the FA_TILE_*
 * classes and records each block's visibility bits (rows and columns of 64 bits).
 * The map depends only on the mask, so one map serves the forward and the backward
 * and every layer that shares the mask. `tiles`: device memory of
 * fa_train_mask_tiles_bytes(p) bytes, 8-byte aligned. Errors: FA_ERR_NULL (no mask,
 * NULL tiles), FA_ERR_ALIGN, the shape and stride errors of the other entry points,
 * FA_ERR_HIP. */
fa_status fa_train_mask_tiles(const fa_attn_params* p, uint8_t* tiles, hipStream_t stream);

/* Static text for a status code. */
const char* fa_train_status_str(fa_status s);
/* Detail text of the calling thread's last error ("" if none). */
const char* fa_train_last_error(void);
/* Gradient of the attention sinks: ADDS, for every query head h,
 *   dsink[h] += -sum_{b, i} exp(sinks[h] - LSE[b, h, i]) * Delta[b, h, i]
 * (the sink is a softmax column with no value, so its dS is P_sink (0 - Delta_i)). LSE and
 * Delta are the forward's and the preprocess's fp32 outputs [B, Hq, Sq] (stride_s 1); a
 * fully masked row has Delta = 0 and adds nothing. dsink: device fp32 [Hq], never zeroed
 * by the library (the caller clears it, or keeps adding as a gradient accumulator). The
 * sum is reduced per workgroup and added with one fp32 atomic per workgroup and head, so
 * its rounding order varies from run to run. Needs p->sinks. */
fa_status fa_train_bwd_sinks(const fa_attn_params* p, const fa_view* lse, const fa_view* delta, float* dsink,
                             hipStream_t stream);

/* q8_0 K/V window (llama.cpp pull request 57 trains a q8_0-quantised cache in place): the
 * rows of a window stored as ggml's q8_0 blocks -- 32 consecutive values along D share
 * one fp16 scale d, each value is the int8 q, the stored value is d * q -- written out as
 * bf16 (one rounding, to nearest even; the fp32 product is exact) into `out`, a bf16 K or V
 * view. The bf16 entry points read such a window in place (kv_format = FA_KV_Q8_0, the same
 * conversion per tile on its way into LDS); this standalone conversion is for callers that
 * want a bf16 copy, and gives the values the in-place walk computes with.
 *   qs : int8 [B, H, S, D] view (element = byte strides), rows 16-byte aligned
 *   d  : fp16 [B, H, S, D / 32] view (element strides), 2-byte aligned, stride_s >= D / 32
 *   out: bf16 [B, H, S, D] view, rows 16-byte aligned; must not overlap qs or d
 * D is 64 or 128. */
fa_status fa_train_dequant_q8_0(int32_t B, int32_t H, int32_t S, int32_t D, const fa_view* qs, const fa_view* d,
                                const fa_view* out, hipStream_t stream);

/* f16 K/V window (llama.cpp pull request 57 trains an f16 cache in place; its backward casts
 * each tile of the cache to F32): the rows of a window stored as IEEE fp16 written out in the
 * compute type of the entry points that read them. out_dtype FA_F32 is exact (every fp16
 * value, subnormals included, is an fp32 value); FA_BF16 rounds to nearest even (bf16 keeps
 * 8 of fp16's 11 significand bits and spans its whole range). The bf16 entry points read an
 * f16 window in place (kv_format = FA_KV_F16); this conversion serves callers that want a copy,
 * such as the fp32 entry points, which read fp32 K / V.
 *   src: fp16 [B, H, S, D] view, rows 16-byte aligned
 *   out: [B, H, S, D] view of out_dtype, rows 16-byte aligned; must not overlap src
 * D is 64 or 128. Errors: FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (D), FA_ERR_DTYPE, the view
 * errors (FA_ERR_NULL, FA_ERR_STRIDE, FA_ERR_ALIGN), FA_ERR_ALIAS, FA_ERR_HIP. */
fa_status fa_train_convert_f16(int32_t B, int32_t H, int32_t S, int32_t D, const fa_view* src, const fa_view* out,
                               int32_t out_dtype, hipStream_t stream);

/* FA_TRAIN_ABI_VERSION of the loaded library. */
int fa_train_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_TRAIN_H */
