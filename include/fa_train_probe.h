/*
 * fa_train_probe.h -- layout probes for the gfx950 matrix-core and LDS-transpose
 * instructions the kernels rely on. Test support, not part of the op.
 *
 * The pages warn that an operand's lane map can differ from the accumulator's and
 * must be derived with a probe kernel, not assumed ("Flash Attn Training" skill
 * page, section 6, trap 10). These entry points run one instruction per wave on
 * caller-chosen register contents and return the raw per-lane results, so a test
 * can derive and assert every lane map the kernels use.
 *
 * All pointers are device pointers; work goes on `stream`; nothing is allocated.
 */
#ifndef FA_TRAIN_PROBE_H
#define FA_TRAIN_PROBE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "fa_train.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_probe_mfma_kind {
    FA_PROBE_MFMA_32X32X16_BF16 = 0, /* a, b: [waves][64][8] (rounded to bf16); c: [waves][64][16] */
    FA_PROBE_MFMA_16X16X32_BF16 = 1, /* a, b: [waves][64][8] (rounded to bf16); c: [waves][64][4]  */
    FA_PROBE_MFMA_32X32X2_F32 = 2,   /* a, b: [waves][64][1];                   c: [waves][64][16] */
    FA_PROBE_MFMA_16X16X4_F32 = 3    /* a, b: [waves][64][1];                   c: [waves][64][4]  */
} fa_probe_mfma_kind;

/* Wave w computes c = MFMA(a[w], b[w], 0) with lane l's operand registers taken from
 * a[w][l][*] and b[w][l][*], and stores lane l's accumulator registers to c[w][l][*].
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (waves < 1 or > 65536, unknown kind), FA_ERR_HIP. */
fa_status fa_train_probe_mfma(int32_t kind, int32_t waves, const float* a, const float* b, float* c,
                              hipStream_t stream);

/* LDS transpose read (ds_read_b64_tr_b16). The kernel fills 8 KiB of LDS with the
 * 16-bit values 0, 1, ..., 4095 (value = element index); lane l of wave w then issues
 * one transpose read at byte address byte_addr[w][l] and stores its four 16-bit
 * results to out[w][l][0..3]. Every address must be a multiple of 8 in [0, 8184]; the
 * kernel reads address 0 instead of any other and reports 0xFFFF in that lane's four
 * results. Errors: FA_ERR_NULL, FA_ERR_SHAPE (waves < 1 or > 4096), FA_ERR_HIP. */
fa_status fa_train_probe_ds_read_tr16(int32_t waves, const int32_t* byte_addr, uint16_t* out,
                                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_TRAIN_PROBE_H */
