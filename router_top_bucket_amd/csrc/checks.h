// Host-side argument checks shared by the C-ABI entry points.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

// The checks of moe_layer_mxfp4: MOE_OK or the status that call returns.
int moe_layer_check(const void *x, moe_dtype x_dtype, const float *w_router, const float *logits, int32_t M,
                    int32_t k, const moe_experts *W, const int32_t *topk_ids, const float *topk_w,
                    const int32_t *offsets, const int32_t *perm, const int32_t *active, const int32_t *n_active,
                    const int32_t *dev_error, const float *y_slots, const float *out, const void *workspace,
                    size_t workspace_bytes);

// Enqueues one layer pass (moe_layer_mxfp4's kernels) once its arguments have
// passed moe_layer_check; workspace holds at least moe_workspace_bytes(M, k, W).
int moe_layer_enqueue(const void *x, moe_dtype x_dtype, const float *w_router, float *logits, int32_t M, int32_t k,
                      const moe_experts *W, int32_t *topk_ids, float *topk_w, int32_t *offsets, int32_t *perm,
                      int32_t *active, int32_t *n_active, int32_t *dev_error, float *y_slots, float *out,
                      void *workspace, void *stream);
