// gemv_bf16.hip -- dense BF16 GEMV for decode, y = W x, B <= 8 rows of x.
//
// "Beating llama.cpp from Scratch on Consumer AMD" (The Optimization Passes,
// Pass 3 item 2) replaces GEMM tiles, which use their tiles poorly at M = 1,
// with a matrix-vector kernel whose vector loads stream the weights; its
// Act 6 shows that decode then sits on the memory-bandwidth wall.  On gfx950
// the same bound applies at ~8 TB/s of HBM3E, so the kernel is shaped only
// around the weight stream:
//  - one wave64 owns R whole rows; lane l reads 16-byte chunks l, l+64, ...
//    of every row (8 bf16 per 128-bit load, 1 KiB per wave instruction,
//    fully coalesced), non-temporal so x stays cached;
//  - x is read through the L1/L2 (a few KiB, shared by every wave); each
//    x chunk is loaded once and reused for the R rows of the wave;
//  - no LDS and no MFMA: at B <= 8 the work is a matvec, bound by HBM;
//  - each (row, b) sum runs over the same lanes and the same chunk order for
//    every B, R and unroll, so a B-row call reproduces the 1-row call bit for
//    bit; the 64 lane partials are combined by a fixed xor butterfly.
#include "common.hpp"
#include "launch.hpp"

namespace mmv {

__device__ __forceinline__ float dot8_bf16(u32x4 w, f32x4 xa, f32x4 xb, float acc) {
  acc = fmaf(bf16_lo(w.x), xa.x, acc);
  acc = fmaf(bf16_hi(w.x), xa.y, acc);
  acc = fmaf(bf16_lo(w.y), xa.z, acc);
  acc = fmaf(bf16_hi(w.y), xa.w, acc);
  acc = fmaf(bf16_lo(w.z), xb.x, acc);
  acc = fmaf(bf16_hi(w.z), xb.y, acc);
  acc = fmaf(bf16_lo(w.w), xb.z, acc);
  acc = fmaf(bf16_hi(w.w), xb.w, acc);
  return acc;
}

// B activation rows, R weight rows per wave, U chunk iterations per
// unrolled step.  256 threads = 4 waves per workgroup.
template <int B, int R, int U>
__global__ __launch_bounds__(256) void k_gemv_bf16(
    const uint16_t *__restrict__ W, int N, int K, int64_t ldw,
    const float *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int row0 = wave * R;
  if (row0 >= N) return;
  const int nch = K >> 3;        // 16-byte chunks per row
  const int nfull = nch >> 6;    // chunk steps where all 64 lanes load

  const uint8_t *wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, N - 1);  // rows past N are computed, not stored
    wrow[r] = reinterpret_cast<const uint8_t *>(W + (int64_t)row * ldw);
  }
  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  int c = lane;
  int it = 0;
  for (; it + U <= nfull; it += U) {
    u32x4 w[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
        w[u][r] = load_stream16(wrow[r] + (int64_t)(c + 64 * u) * 16);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float *xp = X + (int64_t)b * ldx + 8 * (c + 64 * u);
        const f32x4 xa = load_f4(xp), xb = load_f4(xp + 4);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][b] = dot8_bf16(w[u][r], xa, xb, acc[r][b]);
      }
    }
    c += 64 * U;
  }
  // remaining full steps, then the ragged tail (lanes past the row idle)
  for (; it < nfull + 1; ++it) {
    if (c < nch) {
      u32x4 w[R];
#pragma unroll
      for (int r = 0; r < R; ++r) w[r] = load_stream16(wrow[r] + (int64_t)c * 16);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float *xp = X + (int64_t)b * ldx + 8 * c;
        const f32x4 xa = load_f4(xp), xb = load_f4(xp + 4);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][b] = dot8_bf16(w[r], xa, xb, acc[r][b]);
      }
    }
    c += 64;
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = group_sum<64>(acc[r][b]);
      if (lane == 0 && row0 + r < N) Y[(int64_t)b * ldy + row0 + r] = v;
    }
  }
}

template <int B, int R, int U>
static hipError_t launch_bf16(const uint16_t *W, int N, int K, int64_t ldw,
                              const float *X, int64_t ldx, float *Y, int64_t ldy,
                              hipStream_t s) {
  const int waves = (N + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((k_gemv_bf16<B, R, U>), dim3(blocks), dim3(256), 0, s,
                     W, N, K, ldw, X, ldx, Y, ldy);
  return hipGetLastError();
}

hipError_t run_gemv_bf16(const uint16_t *W, int N, int K, int64_t ldw,
                         const float *X, int64_t ldx, int B, float *Y, int64_t ldy,
                         hipStream_t s) {
  switch (B) {
    case 1:
      if (N >= 8192) return launch_bf16<1, 4, 4>(W, N, K, ldw, X, ldx, Y, ldy, s);
      if (N >= 4096) return launch_bf16<1, 2, 4>(W, N, K, ldw, X, ldx, Y, ldy, s);
      return launch_bf16<1, 1, 4>(W, N, K, ldw, X, ldx, Y, ldy, s);
    case 2: return launch_bf16<2, 2, 2>(W, N, K, ldw, X, ldx, Y, ldy, s);
    case 3: return launch_bf16<3, 2, 2>(W, N, K, ldw, X, ldx, Y, ldy, s);
    case 4: return launch_bf16<4, 2, 2>(W, N, K, ldw, X, ldx, Y, ldy, s);
    case 5: return launch_bf16<5, 4, 1>(W, N, K, ldw, X, ldx, Y, ldy, s);
    case 6: return launch_bf16<6, 4, 1>(W, N, K, ldw, X, ldx, Y, ldy, s);
    case 7: return launch_bf16<7, 4, 1>(W, N, K, ldw, X, ldx, Y, ldy, s);
    case 8: return launch_bf16<8, 4, 1>(W, N, K, ldw, X, ldx, Y, ldy, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mmv
