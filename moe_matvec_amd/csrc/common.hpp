// common.hpp -- device helpers shared by the gfx950 kernels.
//
// wave64 throughout: a "lane group" is G consecutive lanes of one wave
// (G in {8, 16, 32, 64}); group reductions are xor butterflies, so every
// lane of the group ends with the same, order-fixed result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmv {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming 128-bit load of data read exactly once (weights): non-temporal
// hint so it does not evict the reused activations from the caches.
__device__ __forceinline__ u32x4 load_stream16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ uint16_t load_stream2(const uint16_t *p) {
  return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ f32x4 load_f4(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}

// bfloat16 pair packed in a dword -> two fp32 values (exact widening)
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return (float)v;
}
// round to nearest even (v_cvt_f16_f32 in the default rounding mode)
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 v = (_Float16)f;
  return __builtin_bit_cast(uint16_t, v);
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
template <int G>
__device__ __forceinline__ int group_sum_i(int v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

}  // namespace mmv
