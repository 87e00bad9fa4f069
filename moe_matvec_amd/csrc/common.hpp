// common.hpp -- device helpers shared by the gfx950 kernels.
//
// wave64 throughout: a "lane group" is G consecutive lanes of one wave
// (G in {8, 16, 32, 64}); group reductions are xor butterflies, so every
// lane of the group ends with the same, order-fixed result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmv {

constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

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

// ---- DPP lane exchanges (no LDS traffic) --------------------------------
// quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror: after these
// four steps every lane of a 16-lane row has combined all 16 values.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Full row and bank masks with in-row permutations: every lane is written
// from a valid source lane, so `old` and bound_ctrl never take effect; the
// form (old = 0, bound_ctrl) lets the compiler fold the move into the DPP
// operand of the instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// sum over each 16-lane row, result in every lane of the row (fixed order)
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  return v;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64_step(uint64_t k) {
  const uint32_t hi = dpp_u32<CTRL>((uint32_t)(k >> 32));
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)k);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > k ? o : k;
}

// maximum over the whole wave, returned in every lane (wave-uniform)
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  k = dpp_max_u64_step<kDppQuadXor1>(k);
  k = dpp_max_u64_step<kDppQuadXor2>(k);
  k = dpp_max_u64_step<kDppRowHalfMirror>(k);
  k = dpp_max_u64_step<kDppRowMirror>(k);
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 16 * r);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 16 * r);
    const uint64_t v = ((uint64_t)hi << 32) | lo;
    best = v > best ? v : best;
  }
  return best;
}

// 8-lane groups (aligned): two quad steps and a half-row mirror
__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  return v;
}
__device__ __forceinline__ float group8_sum(float v) {  // same value in all 8 lanes
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  return v;
}
__device__ __forceinline__ int group8_sum_i(int v) {
  v += (int)dpp_u32<kDppQuadXor1>((uint32_t)v);
  v += (int)dpp_u32<kDppQuadXor2>((uint32_t)v);
  v += (int)dpp_u32<kDppRowHalfMirror>((uint32_t)v);
  return v;
}

// sum over the whole wave: 16-lane rows by DPP, then the four row sums in a
// fixed order; every lane gets the same value
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}
// sum over aligned 32-lane halves
__device__ __forceinline__ float half_sum(float v) {
  v = row16_sum(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (threadIdx.x & 32) ? (c + d) : (a + b);
}
// group sum for G in {16, 32, 64}, every lane of the group gets the sum
template <int G>
__device__ __forceinline__ float gsum(float v) {
  if constexpr (G == 16) return row16_sum(v);
  else if constexpr (G == 32) return half_sum(v);
  else return wave_sum(v);
}

// The same sums, bit for bit, left only in the last lane of each group
// (lane G-1 of it): the row sums are combined by the row-broadcast DPP
// steps (lane 15 of a row into the next row, lane 31 into rows 2 and 3)
// instead of through scalar registers.  Floating-point addition is
// commutative, so (r1 + r0) here equals (r0 + r1) in half_sum, and
// (r3 + r2) + (r1 + r0) equals wave_sum's (r0 + r1) + (r2 + r3).
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows_or_zero(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_rows_or_zero_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
// maximum of a uint32 over the wave, returned wave-uniform (lane 63's value
// after the row and row-broadcast steps)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  v = max(v, dpp_u32<kDppQuadXor2>(v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  v = max(v, dpp_u32<kDppRowMirror>(v));
  v = max(v, dpp_rows_or_zero_u32<kDppRowBcast15, 0xA>(v));
  v = max(v, dpp_rows_or_zero_u32<kDppRowBcast31, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int G>
__device__ __forceinline__ float gsum_last(float v) {
  v = row16_sum(v);
  if constexpr (G >= 32) v += dpp_rows_or_zero<kDppRowBcast15, 0xA>(v);
  if constexpr (G == 64) v += dpp_rows_or_zero<kDppRowBcast31, 0xC>(v);
  return v;
}
__device__ __forceinline__ float wave_sum_last(float v) { return gsum_last<64>(v); }

// gsum_last over N independent values, one reduction step across all of
// them at a time, so that each DPP read is separated from the write of its
// source by independent work rather than by wait states.  Same sums, bit for
// bit, as N calls of gsum_last<G>.
template <int G, int N>
__device__ __forceinline__ void gsum_last_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<kDppQuadXor1>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<kDppQuadXor2>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<kDppRowHalfMirror>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<kDppRowMirror>(v[i]);
  if constexpr (G >= 32) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_rows_or_zero<kDppRowBcast15, 0xA>(v[i]);
  }
  if constexpr (G == 64) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_rows_or_zero<kDppRowBcast31, 0xC>(v[i]);
  }
}

// Order-preserving map of fp32 onto uint32 (larger float, larger key), with
// -0 and +0 mapped to the same key so that they tie; and its inverse.
// Finite inputs map to keys > 0.
__device__ __forceinline__ uint32_t topk_ord(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);  // -0 + 0 = +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float topk_unord(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

}  // namespace mmv
