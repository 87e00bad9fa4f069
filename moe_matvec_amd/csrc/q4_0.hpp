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
  int dot = sdot4((int)(w.x & m), xa.x, -8 * xsum);  // exact: |I| <= 32 * 8 * 127
  dot = sdot4((int)(w.y & m), xa.y, dot);
  dot = sdot4((int)(w.z & m), xa.z, dot);
  dot = sdot4((int)(w.w & m), xa.w, dot);
  dot = sdot4((int)((w.x >> 4) & m), xb.x, dot);
  dot = sdot4((int)((w.y >> 4) & m), xb.y, dot);
  dot = sdot4((int)((w.z >> 4) & m), xb.z, dot);
  dot = sdot4((int)((w.w >> 4) & m), xb.w, dot);
  return dot;
}

// Activations staged in LDS for nrows rows of K (K % 32 == 0):
//   codes int8 [nrows][2][K/2] | d fp32 [nrows][K/32] | qsum int32 [nrows][K/32]
// Each row's codes are two half-planes: bytes 0..15 of every block (block j
// at 16 j), then bytes 16..31.  Lanes that read consecutive blocks then read
// consecutive 16-byte words, which the LDS serves without bank conflicts.
struct XStage {
  int8_t *codes;
  float *d;
  int *qsum;
};
__device__ __forceinline__ size_t xstage_code_off(int r, int K, int j, int byte) {
  return (size_t)r * K + (size_t)(byte >> 4) * (K >> 1) + 16 * j + (byte & 15);
}
__device__ __forceinline__ i32x4 xstage_lo(XStage st, int r, int K, int j) {
  return *reinterpret_cast<const i32x4 *>(st.codes + (size_t)r * K + 16 * j);
}
__device__ __forceinline__ i32x4 xstage_hi(XStage st, int r, int K, int j) {
  return *reinterpret_cast<const i32x4 *>(st.codes + (size_t)r * K + (K >> 1) + 16 * j);
}
// row of task t (0 <= t < nrows * per_row) of a row-major [nrows][per_row]
// task array: no division for one or two rows (nrows is a constant where the
// GEMV kernels inline this)
__device__ __forceinline__ int stage_row(int t, int per_row, int nrows) {
  return nrows == 1 ? 0 : nrows == 2 ? (t >= per_row ? 1 : 0) : t / per_row;
}
// LDS offset of 16-byte chunk c of a row-major [nrows][K] code buffer
__device__ __forceinline__ size_t xstage_chunk_off(int c, int K, int nrows) {
  const int nb = K >> 5, r = stage_row(c, 2 * nb, nrows), rem = c - r * 2 * nb;
  return (size_t)r * K + (size_t)(rem & 1) * (K >> 1) + 16 * (rem >> 1);
}
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

// Two-phase staging for callers that also prefetch weights: loads complete
// in issue order, so the activation loads are issued first (xpre_load), the
// weight loads next, and the quantization (xpre_quantize) then waits only
// for the activations.  One pass covers MAXT tasks (4 floats each) per
// thread, tasks base + threadIdx.x + i * nth (nth: the workgroup's thread
// count, 0 = blockDim.x; a constant lets the index math fold).  Loads are
// unconditional (clamped to the last task) so that they all issue back to
// back; only the stores are guarded.  rowmap == nullptr means rows
// 0..nrows-1, else stage row r holds X row rowmap[r].
template <int MAXT>
struct XPre {
  f32x4 v[MAXT];
};
template <int MAXT>
__device__ __forceinline__ void xpre_load(const float *__restrict__ X, int64_t ldx,
                                          const int *rowmap, int nrows, int K, XPre<MAXT> &p,
                                          int base = 0, int nth = 0) {
  const int nb = K >> 5, total = nrows * nb * 8;
  if (nth == 0) nth = blockDim.x;
#pragma unroll
  for (int i = 0; i < MAXT; ++i) {
    const int t = min(base + (int)threadIdx.x + i * nth, total - 1);
    const int r = stage_row(t, nb * 8, nrows);
    const int rem = t - r * nb * 8;
    const int row = rowmap ? rowmap[r] : r;
    p.v[i] = load_f4(X + (int64_t)row * ldx + 4 * rem);
  }
}
template <int MAXT>
__device__ __forceinline__ void xpre_quantize(const XPre<MAXT> &p, int nrows, int K, XStage st,
                                              int base = 0, int nth = 0) {
  const int nb = K >> 5, total = nrows * nb * 8;
  if (nth == 0) nth = blockDim.x;
  // an unconditional use of every loaded value keeps each load where it was
  // issued (ahead of any later weight loads) instead of letting the
  // compiler sink it into the guarded block below
#pragma unroll
  for (int i = 0; i < MAXT; ++i) asm volatile("" ::"v"(p.v[i]));
#pragma unroll
  for (int i = 0; i < MAXT; ++i) {
    const int t = base + (int)threadIdx.x + i * nth;
    if (t < total) {  // uniform over each 8-lane group: total % 8 == 0
      const Q8Block q = q8_1_quantize8(p.v[i]);
      const int r = stage_row(t, nb * 8, nrows);
      const int rem = t - r * nb * 8;
      const int j = rem >> 3, s = rem & 7;
      *reinterpret_cast<uint32_t *>(st.codes + xstage_code_off(r, K, j, 4 * s)) = q.codes;
      if (s == 0) {
        st.d[r * nb + j] = f16_bits_to_f32(q.d16);
        st.qsum[r * nb + j] = q.qsum;
      }
    }
  }
}

// Quantize rows of fp32 X into the stage, pass after pass of XPre loads
// (all threads of the workgroup call this; blockDim.x % 64 == 0).  `from`
// skips tasks an earlier xpre_load / xpre_quantize pair already covered.
constexpr int kStageMaxT = 8;
template <int PASS = kStageMaxT>  // tasks per thread per pass (registers held: 4 * PASS)
__device__ __forceinline__ void stage_quantize(const float *__restrict__ X, int64_t ldx,
                                               const int *rowmap, int nrows, int K,
                                               XStage st, int from = 0, int nth = 0) {
  const int total = nrows * (K >> 5) * 8;
  if (nth == 0) nth = blockDim.x;
  for (int base = from; base < total; base += PASS * nth) {
    XPre<PASS> p;
    xpre_load(X, ldx, rowmap, nrows, K, p, base, nth);
    xpre_quantize(p, nrows, K, st, base, nth);
  }
}

// The same two phases for a planar Q8_1 buffer (B rows of K codes, then
// B * K/32 {d, s} fp16 pairs): a task is 16 code bytes (half a block), the
// two halves of a block sit in adjacent lanes, and the block's integer code
// sum is formed from both.
template <int MAXC>
struct XqPre {
  i32x4 c[MAXC];
  uint32_t ds[MAXC];
};
template <int MAXC>
__device__ __forceinline__ void xq_pre_load(const uint8_t *__restrict__ Xq, int B, int nrows,
                                            int K, XqPre<MAXC> &p, int base = 0, int nth = 0) {
  const int nb = K >> 5, total = nrows * nb * 2;
  const uint32_t *ds = reinterpret_cast<const uint32_t *>(Xq + (size_t)B * K);
  if (nth == 0) nth = blockDim.x;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int t = min(base + (int)threadIdx.x + i * nth, total - 1);
    p.c[i] = *reinterpret_cast<const i32x4 *>(Xq + (size_t)16 * t);
    p.ds[i] = ds[t >> 1];
  }
}
template <int MAXC>
__device__ __forceinline__ void xq_pre_store(const XqPre<MAXC> &p, int nrows, int K, XStage st,
                                             int base = 0, int nth = 0) {
  const int nb = K >> 5, total = nrows * nb * 2;
  if (nth == 0) nth = blockDim.x;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int t = base + (int)threadIdx.x + i * nth;
    int sum = sdot4(p.c[i].x, 0x01010101, 0);
    sum = sdot4(p.c[i].y, 0x01010101, sum);
    sum = sdot4(p.c[i].z, 0x01010101, sum);
    sum = sdot4(p.c[i].w, 0x01010101, sum);
    sum += (int)dpp_u32<kDppQuadXor1>((uint32_t)sum);  // the block's other half
    // an unconditional use keeps the scale load where it was issued
    uint32_t dsv = p.ds[i];
    asm volatile("" : "+v"(dsv));
    if (t < total) {  // uniform over each lane pair: total is even
      *reinterpret_cast<i32x4 *>(st.codes + xstage_chunk_off(t, K, nrows)) = p.c[i];
      if ((t & 1) == 0) {
        st.d[t >> 1] = f16_bits_to_f32((uint16_t)(dsv & 0xFFFFu));
        st.qsum[t >> 1] = sum;
      }
    }
  }
}
constexpr int kStageMaxC = 8;
__device__ __forceinline__ void stage_copy_q8(const uint8_t *__restrict__ Xq, int B, int nrows,
                                              int K, XStage st, int from = 0, int nth = 0) {
  const int total = nrows * (K >> 5) * 2;
  if (nth == 0) nth = blockDim.x;
  for (int base = from; base < total; base += kStageMaxC * nth) {
    XqPre<kStageMaxC> p;
    xq_pre_load(Xq, B, nrows, K, p, base, nth);
    xq_pre_store(p, nrows, K, st, base, nth);
  }
}

}  // namespace mmv
