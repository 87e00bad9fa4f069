// layout.hpp -- byte sizes and offsets of the library's buffers, shared by
// the host ABI layer and the kernels (host + device inline, no HIP calls).
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifndef __HIPCC__
#define MMV_HD inline
#else
#define MMV_HD __host__ __device__ inline
#endif

namespace mmv {

constexpr size_t kWsAlign = 256;

MMV_HD size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// planar Q8_1: codes [B][K] then {d, s} fp16 pairs [B][K/32]
MMV_HD size_t q8_1_bytes(int K, int B) { return (size_t)B * K + (size_t)4 * B * (K / 32); }

// Q8_1 of h for P pairs, followed by an internal {fp32 d, integer code sum}
// record per block (8 bytes) that the down kernel reads in one load
MMV_HD size_t hq_bytes(int P, int I) { return q8_1_bytes(I, P) + (size_t)8 * P * (I / 32); }

// moe workspace: [hq][gather lists][logits B x (E+1)][ids B x k]
// [weights B x k][shared_w B][per-pair down products P x H fp32]
// [gate/up work items (B > 8): a 32-byte count slot, then at most
//  B*k + B/8 + 1 records of 32 bytes (kWorkRecInts int32 each)]
constexpr int kWorkRecInts = 8;  // one gate/up work record: 32 bytes
struct MoeWsLayout {
  size_t hq, gather, logits, ids, weights, shared_w, dpart, work, total;
};
MMV_HD MoeWsLayout moe_ws_layout(int E, int H, int I, int k, int B, bool has_shared) {
  MoeWsLayout l;
  const int P = B * k + (has_shared ? B : 0);
  l.hq = 0;
  l.gather = align_up(hq_bytes(P, I), kWsAlign);
  l.logits = align_up(l.gather + (size_t)4 * (3 * B * k + 2), kWsAlign);
  l.ids = align_up(l.logits + (size_t)4 * B * (E + 1), kWsAlign);
  l.weights = align_up(l.ids + (size_t)4 * B * k, kWsAlign);
  l.shared_w = align_up(l.weights + (size_t)4 * B * k, kWsAlign);
  l.dpart = align_up(l.shared_w + (size_t)4 * B, kWsAlign);
  l.work = align_up(l.dpart + (size_t)4 * P * H, kWsAlign);
  l.total = align_up(l.work + (size_t)4 * kWorkRecInts * (B * k + B / 8 + 2), kWsAlign);
  return l;
}

// activations staged in LDS by the Q4_0 kernels: codes + d + qsum per block
MMV_HD size_t xstage_lds_bytes(int nrows, int K) {
  return (size_t)nrows * K + (size_t)8 * nrows * (K / 32);
}
constexpr size_t kMaxXStageLds = 64 * 1024;
// the down kernel stages Q8_1(h) of all P pairs in LDS: P * I limit
constexpr int kMaxDownStageElems = 49152;

}  // namespace mmv
