/*
 * fa_train_check.h -- the checked build of the library (libfa_train_check.so, compiled with
 * -DFA_CHECK): debug support, not part of the op.
 *
 * In the checked build every bf16 forward and backward call first verifies, on the host, the
 * index space of the launches it is about to make -- the split choices and workspace layout,
 * every workgroup's unit (tile, batch, head, split) decoded with the kernels' own helpers, the
 * query rows and key tiles each one walks and stages, the LDS offsets of the swizzled tiles, the
 * rows it stores and the workspace slices it writes -- and returns FA_ERR_HIP with
 * "FA_CHECK: ..." in fa_train_last_error() instead of launching when anything falls outside its
 * buffer or an output row is not covered exactly once (once per split).
 */
#ifndef FA_TRAIN_CHECK_H
#define FA_TRAIN_CHECK_H

#include <stddef.h>
#include <stdint.h>

#include "fa_train.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Runs the checker over the bf16 forward's and backward's launches for p, without launching
 * anything (no device needed). key_len_host / q_len_host: host copies of the structured
 * lengths ([B] int32), or NULL for the full lengths. Returns FA_OK, FA_ERR_HIP with the first
 * violation written to report (report_len bytes, NUL-terminated), or the parameter errors of
 * the other entry points; FA_ERR_UNSUPPORTED for fp32 problems. */
fa_status fa_train_check_launch(const fa_attn_params* p, const int32_t* key_len_host, const int32_t* q_len_host,
                                char* report, size_t report_len);

#ifdef __cplusplus
}
#endif

#endif /* FA_TRAIN_CHECK_H */
