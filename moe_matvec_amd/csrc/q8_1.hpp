// q8_1.hpp -- the one device routine that turns fp32 activations into Q8_1.
//
// Used by the standalone quantize_q8_1 kernel, by the activation prologue of
// the Q4_0 GEMV and the expert gate/up kernel, and by the gate/up epilogue
// that quantizes silu(gate)*up ("Fourteen hours to 100 tokens per second",
// Eight levers that worked: Q8 epilogue in the gated kernel).  Because all
// of them call this routine, their codes are bit-identical.
//
// Block rule (32 values x_i):  amax = max|x_i|;  d32 = amax / 127 in fp32
// (correctly rounded division); a block whose fp16 scale rounds to zero is
// stored as all zeros; otherwise q_i = clamp(roundf(x_i * (1/d32)), +-127)
// (roundf: halves away from zero), d = fp16(d32), s = fp16(d32 * sum q_i).
#pragma once

#include "common.hpp"

namespace mmv {

struct Q8Block {
  uint32_t codes;  // this lane's 4 codes, byte t = code (4*s + t)
  uint16_t d16;    // fp16 bits of the block scale   (same in all 8 lanes)
  uint16_t s16;    // fp16 bits of the block sum     (same in all 8 lanes)
  int qsum;        // exact integer sum of the 32 codes
};

__device__ __forceinline__ int q8_code(float x, float id) {
  float t = roundf(__fmul_rn(x, id));
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return (int)t;
}

// One block is held by an aligned group of 8 lanes; lane (lane & 7) = s
// holds values 4s .. 4s+3 of the block in v.  All 8 lanes must be active.
__device__ __forceinline__ Q8Block q8_1_quantize8(f32x4 v) {
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = group8_max(a);
  const float d32 = a / 127.0f;
  const uint16_t d16 = f32_to_f16_bits(d32);
  const bool zero = (d16 & 0x7FFFu) == 0u;
  const float id = zero ? 0.0f : 1.0f / d32;
  const int q0 = q8_code(v.x, id), q1 = q8_code(v.y, id);
  const int q2 = q8_code(v.z, id), q3 = q8_code(v.w, id);
  Q8Block r;
  r.codes = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) |
            ((uint32_t)(q2 & 0xFF) << 16) | ((uint32_t)(q3 & 0xFF) << 24);
  r.qsum = group8_sum_i(q0 + q1 + q2 + q3);
  r.d16 = zero ? (uint16_t)0 : d16;
  // s is the fp16 rounding of the fp32 product d32 * sum q: the product is
  // pinned in a register first, since the compiler otherwise fuses the
  // multiply and the conversion into one instruction that rounds once
  // (v_fma_mixlo_f16), which differs where the fp32 product is an fp16
  // halfway point
  float ps = __fmul_rn(d32, (float)r.qsum);
  asm volatile("" : "+v"(ps));
  r.s16 = zero ? (uint16_t)0 : f32_to_f16_bits(ps);
  return r;
}

}  // namespace mmv
