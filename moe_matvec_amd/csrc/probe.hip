// probe.hip -- device read-bandwidth probe, the yardstick next to the
// 8 TB/s specification ("hanzo-engine: A Portable Single-Binary LLM
// Inference Engine", The Bandwidth Wall: a device roofline probe measures
// the sustainable peak that decode bandwidth is compared against).
// Shaped like the GEMV weight streams it bounds: one-shot workgroups, each
// thread requesting all of its 128-bit non-temporal loads before using any
// (32 KiB per workgroup, contiguous), the words folded with xor so the loads
// cannot be removed, one word per wave written.
#include "common.hpp"
#include "launch.hpp"

namespace mmv {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;  // 16-byte loads per thread
constexpr int kProbeSlots = 8192;
constexpr int64_t kProbeChunk = (int64_t)kProbeThreads * kProbeLoads;  // 16-byte words per workgroup

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const u32x4 *__restrict__ p,
                                                                int64_t n16,
                                                                uint32_t *__restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * kProbeChunk + threadIdx.x;
  u32x4 v[kProbeLoads];
#pragma unroll
  for (int u = 0; u < kProbeLoads; ++u)  // past the end: re-read the last word, not counted
    v[u] = load_stream16(p + min(base + (int64_t)kProbeThreads * u, n16 - 1));
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kProbeLoads; ++u)
    if (base + (int64_t)kProbeThreads * u < n16) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, kWave);
  // the words only keep the loads alive: waves that share a slot overwrite it
  if ((threadIdx.x & 63) == 0)
    out[(blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)) % kProbeSlots] = acc;
}

int probe_slots() { return kProbeSlots; }

hipError_t run_stream_read(const void *buf, size_t bytes, uint32_t *out, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t blocks = (n16 + kProbeChunk - 1) / kProbeChunk;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     reinterpret_cast<const u32x4 *>(buf), n16, out);
  return hipGetLastError();
}

}  // namespace mmv
