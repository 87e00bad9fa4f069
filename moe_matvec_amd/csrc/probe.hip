// probe.hip -- device read-bandwidth probe, the yardstick next to the
// 8 TB/s specification ("hanzo-engine: A Portable Single-Binary LLM
// Inference Engine", The Bandwidth Wall: a device roofline probe measures
// the sustainable peak that decode bandwidth is compared against).
// A grid-stride stream of 128-bit non-temporal loads over a buffer, folded
// with xor so the loads cannot be removed; one word per wave is written.
#include "common.hpp"
#include "launch.hpp"

namespace mmv {

constexpr int kProbeBlocks = 2048;
constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const u32x4 *__restrict__ p,
                                                                int64_t n16,
                                                                uint32_t *__restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = load_stream16(p + i), b = load_stream16(p + i + stride);
    const u32x4 c = load_stream16(p + i + 2 * stride), d = load_stream16(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    acc ^= c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = load_stream16(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, kWave);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

int probe_slots() { return kProbeBlocks * (kProbeThreads / 64); }

hipError_t run_stream_read(const void *buf, size_t bytes, uint32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s,
                     reinterpret_cast<const u32x4 *>(buf), (int64_t)(bytes / 16), out);
  return hipGetLastError();
}

}  // namespace mmv
