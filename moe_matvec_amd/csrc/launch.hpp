// launch.hpp -- internal host-side launchers (one per kernel family).
// Arguments have been validated by the C ABI layer (api.cpp) before these
// are called; each returns hipGetLastError() after its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_matvec.h"
#include "../../include/moe_matvec_testing.h"

namespace mmv {

// value of a kernel-variant switch (moe_matvec_testing.h); 0 = automatic
int path_switch(int which);

// compute units of the current device (queried once per device)
int cu_count();

hipError_t run_gemv_bf16(const uint16_t *W, int N, int K, int64_t ldw,
                         const float *X, int64_t ldx, int B, float *Y, int64_t ldy,
                         hipStream_t s);

hipError_t run_quantize_q8_1(const float *X, int K, int64_t ldx, int B,
                             uint8_t *Xq, hipStream_t s);

hipError_t run_gemv_q4_0(const uint8_t *qs, const uint16_t *d, int N, int K,
                         const float *X, int64_t ldx, const uint8_t *Xq, int B,
                         float *Y, int64_t ldy, hipStream_t s);

hipError_t run_gemv_q4_0_f32(const uint8_t *qs, const uint16_t *d, int N, int K,
                             const float *X, int64_t ldx, int B, float *Y, int64_t ldy,
                             hipStream_t s);

// per-row argmax in two passes; part: B * argmax_parts(N) 64-bit keys
int argmax_parts(int N);
hipError_t run_argmax(const float *Y, int64_t ldy, int N, int B, int32_t *ids, float *vals,
                      uint64_t *part, hipStream_t s);

// router logits (+ shared-gate logit in column E), then top-k and weights
hipError_t run_moe_route(const float *router, int E, int H, const float *X,
                         int64_t ldx, int B, int k, const float *shared_gate_row,
                         float *logits, int32_t *ids, float *weights,
                         float *shared_w, hipStream_t s);

hipError_t run_moe_experts(const mmv_moe_layer &L, const float *X, int64_t ldx,
                           int B, const int32_t *ids, const float *weights,
                           const float *shared_w, float *Y, int64_t ldy,
                           uint8_t *hq, const mmv_moe_debug *dbg, hipStream_t s);

// whole layer in three launches (routing kept on the device)
hipError_t run_moe_layer(const mmv_moe_layer &L, const float *X, int64_t ldx, int B,
                         int32_t *ids, float *weights, float *Y, int64_t ldy, uint8_t *ws,
                         hipStream_t s);

// streaming-read bandwidth probe
int probe_slots();
hipError_t run_stream_read(const void *buf, size_t bytes, uint32_t *out, hipStream_t s);

}  // namespace mmv
