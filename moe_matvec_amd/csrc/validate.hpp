// validate.hpp -- host-side argument checks of the C ABI.  Pure C++: no HIP
// runtime calls, so every error path is testable on a machine without a GPU.
// Each check returns MMV_OK or the first failing mmv_status.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_matvec.h"

namespace mmv {

int check_gemv_bf16(const uint16_t *W, int32_t N, int32_t K, int64_t ldw, const float *X,
                    int64_t ldx, int32_t B, const float *Y, int64_t ldy);
int check_quantize_q8_1(const float *X, int32_t K, int64_t ldx, int32_t B, const void *Xq);
int check_gemv_q4_0(const mmv_q4_0 *W, const float *X, int64_t ldx, const void *Xq,
                    int32_t B, const float *Y, int64_t ldy);
int check_gemv_q4_0_f32(const mmv_q4_0 *W, const float *X, int64_t ldx, int32_t B,
                        const float *Y, int64_t ldy);
size_t argmax_ws_bytes(int32_t N, int32_t B);
int check_argmax(const float *Y, int64_t ldy, int32_t N, int32_t B, const int32_t *ids,
                 const float *vals, const void *ws, size_t ws_bytes);
int check_route(const float *router, int32_t E, int32_t H, const float *X, int64_t ldx,
                int32_t B, int32_t k, const float *shg, const float *logits,
                const int32_t *ids, const float *weights, const float *shared_w);
int check_moe_layer(const mmv_moe_layer *L);
int check_mul_mat_id(const mmv_moe_layer *L, const float *X, int64_t ldx, int32_t B,
                     const int32_t *ids, const float *weights, const float *shared_w,
                     const float *Y, int64_t ldy, const void *ws, size_t ws_bytes);
int check_layer_decode(const mmv_moe_layer *L, const float *X, int64_t ldx, int32_t B,
                       const float *Y, int64_t ldy, const int32_t *ids, const float *weights,
                       const void *ws, size_t ws_bytes);
size_t moe_ws_bytes(const mmv_moe_layer *L, int32_t B);

}  // namespace mmv
