// argmax.hip -- index of the largest value of each row, on the device.
//
// "Beating llama.cpp from Scratch on Consumer AMD" (The Optimization Passes,
// Pass 3 item 3) replaces the copy of the 248,320 logits to the host with an
// on-device parallel argmax, so 4 bytes per token cross the bus.  Here: the
// top-1 case of the routing top-k's ordering.  Each value becomes a 64-bit
// key (order-preserving fp32 bits, -0 = +0, high word; complement of the
// index, low word), so the maximum key is the largest value at its lowest
// index.  Pass 1: a grid of (slices, B) workgroups, each reducing one slice
// of one row with every load issued before the first compare; pass 2: one
// workgroup per row reduces the slices' keys.  Max is exact and
// order-independent: the result does not depend on the slicing.
#include "common.hpp"
#include "launch.hpp"

namespace mmv {

constexpr int kArgSlice = 4096;            // values per pass-1 workgroup
constexpr int kArgPer = kArgSlice / 256;   // per thread, all loads in flight

__device__ __forceinline__ uint64_t argmax_key(float v, int n) {
  return ((uint64_t)topk_ord(v) << 32) | (uint32_t)(~(uint32_t)n);
}

// maximum key of the workgroup (256 threads), valid in thread 0
__device__ __forceinline__ uint64_t block_max_u64(uint64_t k) {
  __shared__ uint64_t wmax[4];
  k = wave_max_u64(k);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = k;
  __syncthreads();
  uint64_t m = wmax[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) m = wmax[w] > m ? wmax[w] : m;
  return m;
}

__global__ __launch_bounds__(256) void k_argmax_part(const float *__restrict__ Y, int64_t ldy,
                                                      int N, uint64_t *__restrict__ part) {
  const int b = blockIdx.y, lo = blockIdx.x * kArgSlice;
  const float *y = Y + (int64_t)b * ldy;
  float v[kArgPer];
#pragma unroll
  for (int m = 0; m < kArgPer; ++m) v[m] = y[min(lo + (int)threadIdx.x + 256 * m, N - 1)];
  uint64_t best = 0;  // below every finite value's key
#pragma unroll
  for (int m = 0; m < kArgPer; ++m) {
    const int n = lo + threadIdx.x + 256 * m;
    const uint64_t k = n < N ? argmax_key(v[m], n) : 0ull;
    best = k > best ? k : best;
  }
  best = block_max_u64(best);
  if (threadIdx.x == 0) part[(int64_t)b * gridDim.x + blockIdx.x] = best;
}

__global__ __launch_bounds__(256) void k_argmax_final(const uint64_t *__restrict__ part,
                                                       int nparts, int32_t *__restrict__ ids,
                                                       float *__restrict__ vals) {
  const int b = blockIdx.x;
  uint64_t best = 0;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    const uint64_t k = part[(int64_t)b * nparts + i];
    best = k > best ? k : best;
  }
  best = block_max_u64(best);
  if (threadIdx.x == 0) {
    ids[b] = (int32_t)(~(uint32_t)best);
    if (vals) vals[b] = topk_unord((uint32_t)(best >> 32));
  }
}

int argmax_parts(int N) { return (N + kArgSlice - 1) / kArgSlice; }

hipError_t run_argmax(const float *Y, int64_t ldy, int N, int B, int32_t *ids, float *vals,
                      uint64_t *part, hipStream_t s) {
  const int np = argmax_parts(N);
  hipLaunchKernelGGL(k_argmax_part, dim3(np, B), dim3(256), 0, s, Y, ldy, N, part);
  hipLaunchKernelGGL(k_argmax_final, dim3(B), dim3(256), 0, s, part, np, ids, vals);
  return hipGetLastError();
}

}  // namespace mmv
