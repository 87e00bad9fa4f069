// q4_0.hpp -- Q4_0 x Q8_1 block arithmetic and activation staging in LDS.
//
// Q4_0 block: 32 weights, fp16 scale d, codes 0..15, weight = d*(code - 8);
// byte i of the 16 code bytes holds code i (low nibble) and code i+16 (high
// nibble), the split-nibble order of the Q4_0 loaders in "Flash-Next on
// Strix Halo" (Correctness fixes).  The product with a Q8_1 block is
//   d_w * d_x * I,   I = sum_i (code_i - 8) q_i = dot(code, q) - 8 * sum(q),
// with I an exact int32: eight v_dot4 on the unpacked nibbles, and sum(q)
// computed once per activation block when it is staged, so the fp16 "s"
// field of Q8_1 is never needed and nothing is rounded before the scale.
#pragma once

#include "common.hpp"
#include "q8_1.hpp"
#include "layout.hpp"

namespace mmv {

// dot of one Q4_0 block's 32 codes (w) with 32 int8 codes (xa: codes 0..15,
// xb: codes 16..31), minus 8 * xsum.
__device__ __forceinline__ int q4_block_isum(u32x4 w, i32x4 xa, i32x4 xb, int xsum) {
  const uint32_t m = 0x0F0F0F0Fu;
  int dot = sdot4((int)(w.x & m), xa.x, 0);
  dot = sdot4((int)(w.y & m), xa.y, dot);
  dot = sdot4((int)(w.z & m), xa.z, dot);
  dot = sdot4((int)(w.w & m), xa.w, dot);
  dot = sdot4((int)((w.x >> 4) & m), xb.x, dot);
  dot = sdot4((int)((w.y >> 4) & m), xb.y, dot);
  dot = sdot4((int)((w.z >> 4) & m), xb.z, dot);
  dot = sdot4((int)((w.w >> 4) & m), xb.w, dot);
  return dot - 8 * xsum;
}

// Activations staged in LDS for nrows rows of K (K % 32 == 0):
//   codes int8 [nrows][K] | d fp32 [nrows][K/32] | qsum int32 [nrows][K/32]
struct XStage {
  int8_t *codes;
  float *d;
  int *qsum;
};
__host__ __device__ inline size_t xstage_bytes(int nrows, int K) {
  return xstage_lds_bytes(nrows, K);
}
__device__ __forceinline__ XStage xstage_at(uint8_t *base, int nrows, int K) {
  XStage s;
  s.codes = reinterpret_cast<int8_t *>(base);
  s.d = reinterpret_cast<float *>(base + (size_t)nrows * K);
  s.qsum = reinterpret_cast<int *>(base + (size_t)nrows * K + (size_t)4 * nrows * (K / 32));
  return s;
}

// Quantize rows rowmap[0..nrows) of fp32 X into the stage (all threads of
// the workgroup call this; blockDim.x % 64 == 0).  rowmap == nullptr means
// rows 0..nrows-1.  Codes are those of q8_1_quantize8.
__device__ __forceinline__ void stage_quantize(const float *__restrict__ X, int64_t ldx,
                                               const int *rowmap, int nrows, int K,
                                               XStage st) {
  const int nb = K >> 5;
  const int total = nrows * nb * 8;
  for (int t = threadIdx.x; t < total; t += blockDim.x) {
    const int r = t / (nb * 8);
    const int rem = t - r * nb * 8;
    const int j = rem >> 3, s = rem & 7;
    const int row = rowmap ? rowmap[r] : r;
    const f32x4 v = load_f4(X + (int64_t)row * ldx + 32 * j + 4 * s);
    const Q8Block q = q8_1_quantize8(v);
    *reinterpret_cast<uint32_t *>(st.codes + (size_t)r * K + 32 * j + 4 * s) = q.codes;
    if (s == 0) {
      st.d[r * nb + j] = f16_bits_to_f32(q.d16);
      st.qsum[r * nb + j] = q.qsum;
    }
  }
}

// Two-phase staging for callers that also prefetch weights: loads complete
// in issue order, so the activation loads are issued first (xpre_load), the
// weight loads next, and the quantization (xpre_quantize) then waits only
// for the activations.  MAXT = tasks per thread (4 floats each) the caller
// guarantees: nrows * K / 4 <= MAXT * blockDim.x.
template <int MAXT>
struct XPre {
  f32x4 v[MAXT];
};
template <int MAXT>
__device__ __forceinline__ void xpre_load(const float *__restrict__ X, int64_t ldx,
                                          const int *rowmap, int nrows, int K, XPre<MAXT> &p) {
  const int nb = K >> 5, total = nrows * nb * 8;
#pragma unroll
  for (int i = 0; i < MAXT; ++i) {
    const int t = threadIdx.x + i * blockDim.x;
    if (t < total) {
      const int r = t / (nb * 8);
      const int rem = t - r * nb * 8;
      const int row = rowmap ? rowmap[r] : r;
      p.v[i] = load_f4(X + (int64_t)row * ldx + 4 * rem);
    }
  }
}
template <int MAXT>
__device__ __forceinline__ void xpre_quantize(const XPre<MAXT> &p, int nrows, int K, XStage st) {
  const int nb = K >> 5, total = nrows * nb * 8;
#pragma unroll
  for (int i = 0; i < MAXT; ++i) {
    const int t = threadIdx.x + i * blockDim.x;
    if (t < total) {  // uniform over each 8-lane group: total % 8 == 0
      const int r = t / (nb * 8);
      const int rem = t - r * nb * 8;
      const int j = rem >> 3, s = rem & 7;
      const Q8Block q = q8_1_quantize8(p.v[i]);
      *reinterpret_cast<uint32_t *>(st.codes + (size_t)r * K + 32 * j + 4 * s) = q.codes;
      if (s == 0) {
        st.d[r * nb + j] = f16_bits_to_f32(q.d16);
        st.qsum[r * nb + j] = q.qsum;
      }
    }
  }
}

// Copy rows of a planar Q8_1 buffer (B rows of K) into the stage.
__device__ __forceinline__ void stage_copy_q8(const uint8_t *__restrict__ Xq, int B,
                                              int nrows, int K, XStage st) {
  const int nb = K >> 5;
  const int total = nrows * nb * 8;
  const uint16_t *ds = reinterpret_cast<const uint16_t *>(Xq + (size_t)B * K);
  for (int t = threadIdx.x; t < total; t += blockDim.x) {
    const int r = t / (nb * 8);
    const int rem = t - r * nb * 8;
    const int j = rem >> 3, s = rem & 7;
    const uint32_t c = *reinterpret_cast<const uint32_t *>(Xq + (size_t)r * K + 32 * j + 4 * s);
    *reinterpret_cast<uint32_t *>(st.codes + (size_t)r * K + 32 * j + 4 * s) = c;
    const int sum = group8_sum_i(sdot4((int)c, 0x01010101, 0));
    if (s == 0) {
      st.d[r * nb + j] = f16_bits_to_f32(ds[((size_t)r * nb + j) * 2]);
      st.qsum[r * nb + j] = sum;
    }
  }
}

}  // namespace mmv
