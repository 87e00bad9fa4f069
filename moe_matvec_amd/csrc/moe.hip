// moe.hip -- the mixture-of-experts decode path: F32 router, softmax +
// top-k, per-expert row lists, gate/up with SiLU and a Q8_1 epilogue, and
// the down projection with the weighted combine and the shared expert.
//
// "Fourteen hours to 100 tokens per second" traces one decode token as
// separate kernel classes (F32 router, top-k routing, mul_mat_id expert
// matvecs, quantize_q8_1, broadcast glue), finds that kernels below five
// microseconds cost more to launch than to run, and removes glue by fusion:
// the top-k kernel writes ids and weights directly, silu(gate)*up is
// quantized to Q8 in the producing kernel, the K <= 512 down projection uses
// four rows per wave.  "Flash-Next on Strix Halo" (Expert GEMMs) builds
// per-expert row lists so each expert's weights are read once for all rows
// that chose it.  Here, on gfx950, one layer is three launches for B <= 2,
// five up to B = 8 and six for the verify / prefill batches above (see the
// section on those):
//  K1 router rows, logits to the workspace (B <= 3: one wave per router row
//     with every activation row in registers, all loads issued up front;
//     B >= 4 with H of 1024 or 2048: workgroups per 8 activation rows, x
//     staged in LDS; the same per-lane order and wave sum either way);
//  (B > 2) K1b one workgroup, a wave per row: top-k with order-preserving
//     32-bit keys (equal logits rank by lower index), weights exp(l - l_max)
//     renormalised over the selected k (the full-E denominator cancels), and
//     the per-expert row lists, published for K2 and K3;
//  K2 gate/up: a workgroup owns 32 rows of one expert's gate and up (the
//     shared expert first, then the unique routed experts; 16 lanes per row,
//     every weight load issued before x is staged as Q8_1 in LDS); for B <= 2
//     every workgroup runs top-k on the logits itself (no extra launch);
//     silu(g)*u in registers; the tile's 32 h values are exactly one Q8_1
//     block of the down input, quantized in the epilogue;
//  K3 down + combine (B <= 2): a workgroup owns 4 output rows (16 lanes per
//     row, one Q4_0 block per lane at I = 512); its waves split the experts
//     by expert id; each (row, pair) product is formed whole (per lane its
//     blocks, then the 16-lane sum) and a row's pairs are added by a fixed
//     tree over its slots, then the shared expert's term: no atomics, one
//     store per output;
//  K3 by expert + K4 combine (B >= 3): a workgroup owns one expert and 64
//     output rows and writes each of its pairs' products (the same values,
//     bit for bit) to the workspace; K4 adds them with the same tree.
//  Every row's result is thus the same bits for every B.
// A grid-wide barrier inside one kernel measured slower than a launch
// boundary on this GPU, so the phases stay separate launches.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "layout.hpp"
#include "q4_0.hpp"
#include "q8_1.hpp"

namespace mmv {

constexpr int kMaxPairs = MMV_MAX_BATCH * MMV_MAX_TOPK;  // 128

// ---------------------------------------------------------------------------
// Timeline build (-DMMV_TIMELINE, a separate library for measurement): thread
// 0 of every workgroup of the MoE kernels notes the chip's constant 100 MHz
// clock (s_memrealtime) at fixed points into LDS, and at its end writes them
// to a device array: [kernel kind][workgroup][point].  In the normal build
// the macros are empty.
// ---------------------------------------------------------------------------
enum TlKind { kTlRouter, kTlRouterLds, kTlTopkGather, kTlGateUp, kTlDown, kTlDownPart,
              kTlCombine, kTlKinds };
#ifdef MMV_TIMELINE
constexpr int kTlSlots = 4096, kTlPoints = 8;
__device__ uint64_t g_timeline[kTlKinds][kTlSlots][kTlPoints];
__shared__ uint64_t s_timeline[kTlPoints];
#define MMV_TL(i)                                                                        \
  do {                                                                                   \
    if (threadIdx.x == 0) s_timeline[i] = __builtin_amdgcn_s_memrealtime();             \
  } while (0)
#define MMV_TL_END(kind, i)                                                              \
  do {                                                                                   \
    if (threadIdx.x == 0) {                                                              \
      s_timeline[i] = __builtin_amdgcn_s_memrealtime();                                  \
      if (blockIdx.x < (unsigned)kTlSlots)                                               \
        for (int q_ = 0; q_ <= (i); ++q_) g_timeline[kind][blockIdx.x][q_] = s_timeline[q_]; \
    }                                                                                    \
  } while (0)
#else
#define MMV_TL(i) \
  do {            \
  } while (0)
#define MMV_TL_END(kind, i) \
  do {                      \
  } while (0)
#endif

// ---------------------------------------------------------------------------
// router rows: logits[b * ldl + e] = R[e] . x_b (row E = shared gate row)
// ---------------------------------------------------------------------------
// HC = H / 256 float4 chunks per lane (compile time: every load issued up
// front), or 0 for any H % 4 == 0 (runtime loop).
template <int B, int HC>
__device__ __forceinline__ void router_row(const float *__restrict__ row, int H,
                                           const float *__restrict__ X, int64_t ldx,
                                           float *__restrict__ out, int64_t ldl) {
  const int lane = threadIdx.x & 63;
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  auto step = [&](const f32x4 r, int c) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const f32x4 x = load_f4(X + (int64_t)b * ldx + 4 * c);
      acc[b] = fmaf(r.x, x.x, acc[b]);
      acc[b] = fmaf(r.y, x.y, acc[b]);
      acc[b] = fmaf(r.z, x.z, acc[b]);
      acc[b] = fmaf(r.w, x.w, acc[b]);
    }
  };
  if constexpr (HC > 0) {
    f32x4 r[HC];
#pragma unroll
    for (int i = 0; i < HC; ++i)
      r[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row) + lane + 64 * i);
#pragma unroll
    for (int i = 0; i < HC; ++i) step(r[i], lane + 64 * i);
  } else {
    for (int c = lane; c < (H >> 2); c += 64)
      step(__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row) + c), c);
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float v = wave_sum_last(acc[b]);
    if (lane == 63) out[(int64_t)b * ldl] = v;
  }
}

// ---------------------------------------------------------------------------
// top-k of one row by one wave
// ---------------------------------------------------------------------------
// Selects the k largest of l[0..E) (ties: lower index first), writes ids,
// renormalised weights and the shared weight.  Whole wave, uniform control.
// KPL = keys per lane (E <= 64 * KPL); lane l holds experts l + 64 i, as
// order-preserving keys (-0 = +0; padding lanes hold 0, below every logit).
// Each lane first sorts its own keys, largest first (a min/max network), so
// that a round needs only the lanes' leading keys: the wave maximum M of
// them (DPP), the lane holding it (one ballot; when several lanes hold M,
// the lowest expert index among their leading elements wins), and that lane
// drops its leading key.  Which of a lane's elements a pick was is settled
// after the rounds from the lane's unsorted keys: the lowest index holding M
// that earlier picks of the same lane and value have not taken.  With one
// wave per row the rounds are bound by instruction issue, so what counts is
// a round's instruction count: about 30 + KPL here against about 12 * KPL
// for rescanning every key each round.

// Batcher's odd-even merge sort networks (comparator pairs a[c] < b[c]),
// applied largest first; N a power of two.
template <int N> struct SortNet {
  static constexpr int n = 0;
  static constexpr unsigned char a[1] = {0};
  static constexpr unsigned char b[1] = {0};
};
template <> struct SortNet<2> {
  static constexpr int n = 1;
  static constexpr unsigned char a[1] = {0};
  static constexpr unsigned char b[1] = {1};
};
template <> struct SortNet<4> {
  static constexpr int n = 5;
  static constexpr unsigned char a[5] = {0, 2, 0, 1, 1};
  static constexpr unsigned char b[5] = {1, 3, 2, 3, 2};
};
template <> struct SortNet<8> {
  static constexpr int n = 19;
  static constexpr unsigned char a[19] = {0, 2, 4, 6, 0, 1, 4, 5, 1, 5, 0, 1, 2, 3, 2, 3, 1, 3, 5};
  static constexpr unsigned char b[19] = {1, 3, 5, 7, 2, 3, 6, 7, 2, 6, 4, 5, 6, 7, 4, 5, 2, 4, 6};
};
template <> struct SortNet<16> {
  static constexpr int n = 63;
  static constexpr unsigned char a[63] = {0, 2, 4, 6, 8, 10, 12, 14, 0, 1, 4, 5, 8, 9, 12, 13, 1, 5, 9, 13, 0, 1, 2, 3, 8, 9, 10, 11, 2, 3, 10, 11, 1, 3, 5, 9, 11, 13, 0, 1, 2, 3, 4, 5, 6, 7, 4, 5, 6, 7, 2, 3, 6, 7, 10, 11, 1, 3, 5, 7, 9, 11, 13};
  static constexpr unsigned char b[63] = {1, 3, 5, 7, 9, 11, 13, 15, 2, 3, 6, 7, 10, 11, 14, 15, 2, 6, 10, 14, 4, 5, 6, 7, 12, 13, 14, 15, 4, 5, 12, 13, 2, 4, 6, 10, 12, 14, 8, 9, 10, 11, 12, 13, 14, 15, 8, 9, 10, 11, 4, 5, 8, 9, 12, 13, 2, 4, 6, 8, 10, 12, 14};
};

template <int N>
__device__ __forceinline__ void sort_desc_u32(uint32_t (&v)[N]) {
#pragma unroll
  for (int c = 0; c < SortNet<N>::n; ++c) {
    const uint32_t x = v[SortNet<N>::a[c]], y = v[SortNet<N>::b[c]];
    v[SortNet<N>::a[c]] = max(x, y);
    v[SortNet<N>::b[c]] = min(x, y);
  }
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// Slot (0..KPL) of this lane's element that a pick of value M takes: earlier
// picks of this lane with value M took the lowest such slots, and their
// number is the count of M among the unsorted keys minus the count of M
// still in the sorted list.
template <int KPL>
__device__ __forceinline__ int slot_of_value(const uint32_t (&orig)[KPL], int taken, uint32_t M) {
  int seen = 0, s = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const bool m = orig[i] == M;
    s = (m && seen == taken) ? i : s;
    seen += m ? 1 : 0;
  }
  return s;
}

template <int KPL>
__device__ void topk_row(const float *__restrict__ l, int E, int k, int has_shared,
                         int32_t *__restrict__ ids, float *__restrict__ weights,
                         float *__restrict__ shared_w) {
  const int lane = threadIdx.x & 63;
  float v[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) v[i] = l[min(lane + 64 * i, E - 1)];
  const float lsh = has_shared ? l[E] : 0.0f;
  uint32_t orig[KPL], key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    orig[i] = lane + 64 * i < E ? topk_ord(v[i]) : 0u;
    key[i] = orig[i];
  }
  sort_desc_u32<KPL>(key);
  // equal keys within a lane (rare): picks then count earlier picks
  bool dup = false;
#pragma unroll
  for (int i = 0; i + 1 < KPL; ++i) dup = dup || (key[i] == key[i + 1] && key[i] != 0u);
  const bool any_dup = __ballot(dup) != 0ull;

  uint32_t pick_lane = 0, pick_key = 0;  // round j's pick, held by lane j
  for (int j = 0; j < k; ++j) {
    const uint32_t M = wave_max_u32(key[0]);
    const unsigned long long hit = __ballot(key[0] == M);
    uint32_t L;
    if (__popcll(hit) == 1) {
      L = (uint32_t)__builtin_ctzll(hit);
    } else {  // the lowest index among the lanes' leading elements equal to M
      int cnt_o = 0, cnt_r = 0;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        cnt_o += orig[i] == M ? 1 : 0;
        cnt_r += key[i] == M ? 1 : 0;
      }
      const int s = slot_of_value<KPL>(orig, cnt_o - cnt_r, M);
      L = wave_min_u32(key[0] == M ? ((uint32_t)s << 6) | (uint32_t)lane : 0xFFFFFFFFu) & 63u;
    }
    // the winning lane shifts its list by one (bit-select with an opaque
    // mask: written as a select, the compiler rebuilds it as a dynamically
    // indexed vector read)
    uint32_t m = (uint32_t)lane == L ? ~0u : 0u;
    asm volatile("" : "+v"(m));
#pragma unroll
    for (int i = 0; i + 1 < KPL; ++i) key[i] = (key[i + 1] & m) | (key[i] & ~m);
    key[KPL - 1] &= ~m;
    pick_lane = lane == j ? L : pick_lane;
    pick_key = lane == j ? M : pick_key;
  }
  // which element of lane pick_lane each pick was (lanes j < k)
  int taken = 0;
  if (any_dup) {
    for (int j = 0; j < k; ++j) {
      const uint32_t Lj = (uint32_t)__builtin_amdgcn_readlane((int)pick_lane, j);
      const uint32_t Mj = (uint32_t)__builtin_amdgcn_readlane((int)pick_key, j);
      taken += (j < lane && Lj == pick_lane && Mj == pick_key) ? 1 : 0;
    }
  }
  uint32_t theirs[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i)
    theirs[i] = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(pick_lane << 2), (int)orig[i]);
  const int my_id = 64 * slot_of_value<KPL>(theirs, taken, pick_key) + (int)pick_lane;
  const float my_l = lane < k ? topk_unord(pick_key) : 0.0f;

  const float lmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float ex = lane < k ? expf(my_l - lmax) : 0.0f;
  const float den = row16_sum(ex);  // k <= 16: lanes 0..15
  if (lane < k) {
    ids[lane] = my_id;
    weights[lane] = ex / den;
  }
  if (lane == 0 && shared_w) *shared_w = has_shared ? 1.0f / (1.0f + expf(-lsh)) : 1.0f;
}

template <int KPL>
__device__ __forceinline__ void topk_rows(const float *__restrict__ L, int64_t ldl, int E, int B,
                                          int k, int has_shared, int32_t *__restrict__ ids,
                                          float *__restrict__ weights,
                                          float *__restrict__ shared_w) {
  for (int b = threadIdx.x >> 6; b < B; b += blockDim.x >> 6)
    topk_row<KPL>(L + (int64_t)b * ldl, E, k, has_shared, ids + (int64_t)b * k,
                  weights + (int64_t)b * k, shared_w ? shared_w + b : nullptr);
}

// dispatch on the number of experts (keys per lane)
__device__ __forceinline__ void topk_any(const float *__restrict__ L, int64_t ldl, int E, int B,
                                         int k, int has_shared, int32_t *__restrict__ ids,
                                         float *__restrict__ weights,
                                         float *__restrict__ shared_w) {
  if (E <= 64) topk_rows<1>(L, ldl, E, B, k, has_shared, ids, weights, shared_w);
  else if (E <= 256) topk_rows<4>(L, ldl, E, B, k, has_shared, ids, weights, shared_w);
  else if (E <= 512) topk_rows<8>(L, ldl, E, B, k, has_shared, ids, weights, shared_w);
  else topk_rows<16>(L, ldl, E, B, k, has_shared, ids, weights, shared_w);
}

// ---------------------------------------------------------------------------
// moe_route_topk: router kernel (4 rows per workgroup) + one top-k workgroup
// ---------------------------------------------------------------------------
template <int B, int HC>
__global__ __launch_bounds__(256) void k_router(const float *__restrict__ R, int E, int H,
                                                const float *__restrict__ shg,
                                                const float *__restrict__ X, int64_t ldx,
                                                float *__restrict__ logits) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = E + (shg ? 1 : 0);
  if (e >= rows) return;
  const float *row = e < E ? R + (int64_t)e * H : shg;
  router_row<B, HC>(row, H, X, ldx, logits + e, E + 1);
}

// Router rows for B >= 4 (any B <= 64 in one launch): a workgroup per (4 * RW
// router rows, 8 activation rows).  The workgroup stages its 8 rows of x in
// LDS once (each wave holding all B rows of x in registers spills at B = 8
// and leaves one wave per SIMD); a wave owns RW router rows, held in
// registers.  Groups of 8 (or 4) rows run as 8 * RW (4 * RW) independent
// chains side by side (their wave sums too), so no chain waits on its
// predecessor; each x value read from LDS serves RW router rows.  Per lane
// the same fused multiply-adds in the same order as router_row, then the
// same wave sum: the same logits, bit for bit.  Dynamic LDS: 8 * H * 4
// bytes.  HC = H / 256.
template <int HC, int RW>
__global__ __launch_bounds__(256) void k_router_lds(const float *__restrict__ R, int E,
                                                    const float *__restrict__ shg,
                                                    const float *__restrict__ X, int64_t ldx,
                                                    int B, float *__restrict__ logits) {
  extern __shared__ __align__(16) f32x4 xs4[];  // [8][H / 4]
  constexpr int H4 = 64 * HC;                    // float4 per row
  constexpr int PER = 8 * H4 / 256;              // staging float4 per thread
  const int lane = threadIdx.x & 63;
  const int e0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RW;
  const int rows = E + (shg ? 1 : 0);
  const int b0 = blockIdx.y * 8, nb = min(8, B - b0);
  MMV_TL(0);
  f32x4 r[RW][HC];
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    const int e = e0 + j;  // rows past the end read row 0 and store nothing
    const float *row = e < E ? R + (int64_t)e * 4 * H4 : (e == E && shg ? shg : R);
#pragma unroll
    for (int i = 0; i < HC; ++i)
      r[j][i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row) + lane + 64 * i);
  }
  f32x4 xv[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int t = threadIdx.x + 256 * m, bb = min(t / H4, nb - 1), c = t - (t / H4) * H4;
    xv[m] = load_f4(X + (int64_t)(b0 + bb) * ldx + 4 * c);
  }
#pragma unroll
  for (int m = 0; m < PER; ++m) xs4[threadIdx.x + 256 * m] = xv[m];
  __syncthreads();
  MMV_TL_END(kTlRouterLds, 1);  // x staged: the products follow (thread 0's wave)
  if (e0 >= rows) return;  // uniform over the wave; no barrier follows
  auto chain = [&](float &acc, const f32x4 &w, const f32x4 &x) {
    acc = fmaf(w.x, x.x, acc);
    acc = fmaf(w.y, x.y, acc);
    acc = fmaf(w.z, x.z, acc);
    acc = fmaf(w.w, x.w, acc);
  };
  auto put = [&](int bb, int j, float v) {
    if (lane == 63 && e0 + j < rows) logits[(int64_t)(b0 + bb) * (E + 1) + e0 + j] = v;
  };
  // NB rows from g0 as NB * RW chains side by side.  x chunk i + 1 is read
  // while chunk i is used; the scheduling barriers and the opaque
  // accumulators keep the compiler from hoisting every LDS read and running
  // one chain after another (which needs 256 registers of x).
  auto group = [&](auto nbc, int g0) {
    constexpr int NB = decltype(nbc)::value;
    float acc[RW][NB];
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) acc[j][bb] = 0.0f;
    f32x4 xa[NB], xb[NB];
    auto ld = [&](f32x4(&x)[NB], int i) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) x[bb] = xs4[(g0 + bb) * H4 + lane + 64 * i];
    };
    auto mac = [&](const f32x4(&x)[NB], int i) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int j = 0; j < RW; ++j) {
          chain(acc[j][bb], r[j][i], x[bb]);
          asm volatile("" : "+v"(acc[j][bb]));  // the products of chunk i happen here
        }
    };
    static_assert(HC % 2 == 0, "chunks go in pairs");
    ld(xa, 0);
#pragma unroll
    for (int i = 0; i < HC; i += 2) {
      ld(xb, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      mac(xa, i);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 2 < HC) ld(xa, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      mac(xb, i + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    float v[RW][NB];  // every wave sum first, side by side, then the stores
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) v[j][bb] = wave_sum_last(acc[j][bb]);
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) put(g0 + bb, j, v[j][bb]);
  };
  if (nb == 8) {  // uniform
    group(std::integral_constant<int, 8>{}, 0);
    return;
  }
  int g = 0;
  if (nb >= 4) {
    group(std::integral_constant<int, 4>{}, 0);
    g = 4;
  }
  for (int bb = g; bb < nb; ++bb) {  // uniform
    float acc[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      const f32x4 x = xs4[bb * H4 + lane + 64 * i];
#pragma unroll
      for (int j = 0; j < RW; ++j) chain(acc[j], r[j][i], x);
    }
#pragma unroll
    for (int j = 0; j < RW; ++j) put(bb, j, wave_sum_last(acc[j]));
  }
}

// a workgroup per 4 rows (a wave per row)
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ L, int64_t ldl, int E,
                                              int B, int k, int has_shared,
                                              int32_t *__restrict__ ids,
                                              float *__restrict__ weights,
                                              float *__restrict__ shared_w) {
  const int b0 = blockIdx.x * 4;
  topk_any(L + (int64_t)b0 * ldl, ldl, E, min(4, B - b0), k, has_shared, ids + (int64_t)b0 * k,
           weights + (int64_t)b0 * k, shared_w ? shared_w + b0 : nullptr);
}

template <int B>
static void launch_router(const float *router, int E, int H, const float *shg, const float *X,
                          int64_t ldx, float *logits, hipStream_t s) {
  const int rows = E + (shg ? 1 : 0);
  const dim3 grid((rows + 3) / 4), block(256);
  switch (H) {
    case 1024: hipLaunchKernelGGL((k_router<B, 4>), grid, block, 0, s, router, E, H, shg, X, ldx, logits); break;
    case 2048: hipLaunchKernelGGL((k_router<B, 8>), grid, block, 0, s, router, E, H, shg, X, ldx, logits); break;
    case 4096: hipLaunchKernelGGL((k_router<B, 16>), grid, block, 0, s, router, E, H, shg, X, ldx, logits); break;
    default: hipLaunchKernelGGL((k_router<B, 0>), grid, block, 0, s, router, E, H, shg, X, ldx, logits); break;
  }
}

// two router rows per wave from 32 activation rows (E = 512, H = 2048: at 16
// rows one per wave measured 68.2 against 69.4 us per layer; at 64 rows two
// per wave 158.5 against 160.4)
constexpr int kRouterTwoRowsMinB = 32;

// B >= 4 with H of 1024 or 2048: every row in one launch of the LDS-staged
// router (same logits as router_row); returns false when it does not apply
static bool launch_router_lds(const float *router, int E, int H, const float *shg,
                              const float *X, int64_t ldx, int B, float *logits, hipStream_t s) {
  if (B < 4 || (H != 1024 && H != 2048)) return false;
  const int rows = E + (shg ? 1 : 0), gy = (B + 7) / 8;
  const dim3 block(256), grid1((rows + 3) / 4, gy), grid2((rows + 7) / 8, gy);
  const size_t lds = (size_t)8 * H * 4;
  // two router rows per wave once there are workgroups enough for the chip
  const bool two = B >= kRouterTwoRowsMinB;
  if (H == 1024) {
    if (two)
      hipLaunchKernelGGL((k_router_lds<4, 2>), grid2, block, lds, s, router, E, shg, X, ldx, B, logits);
    else
      hipLaunchKernelGGL((k_router_lds<4, 1>), grid1, block, lds, s, router, E, shg, X, ldx, B, logits);
  } else {
    if (two)
      hipLaunchKernelGGL((k_router_lds<8, 2>), grid2, block, lds, s, router, E, shg, X, ldx, B, logits);
    else
      hipLaunchKernelGGL((k_router_lds<8, 1>), grid1, block, lds, s, router, E, shg, X, ldx, B, logits);
  }
  return true;
}

hipError_t run_moe_route(const float *router, int E, int H, const float *X, int64_t ldx,
                         int B, int k, const float *shg, float *logits, int32_t *ids,
                         float *weights, float *shared_w, hipStream_t s) {
  const float *L = X;
  int64_t ldl = ldx;
  if (router && !launch_router_lds(router, E, H, shg, X, ldx, B, logits, s)) {
    for (int b0 = 0; b0 < B; b0 += MMV_MAX_BATCH) {  // router rows 8 activation rows at a time
      const float *Xc = X + (int64_t)b0 * ldx;
      float *lc = logits + (int64_t)b0 * (E + 1);
      switch (min(B - b0, MMV_MAX_BATCH)) {
        case 1: launch_router<1>(router, E, H, shg, Xc, ldx, lc, s); break;
        case 2: launch_router<2>(router, E, H, shg, Xc, ldx, lc, s); break;
        case 3: launch_router<3>(router, E, H, shg, Xc, ldx, lc, s); break;
        case 4: launch_router<4>(router, E, H, shg, Xc, ldx, lc, s); break;
        case 5: launch_router<5>(router, E, H, shg, Xc, ldx, lc, s); break;
        case 6: launch_router<6>(router, E, H, shg, Xc, ldx, lc, s); break;
        case 7: launch_router<7>(router, E, H, shg, Xc, ldx, lc, s); break;
        case 8: launch_router<8>(router, E, H, shg, Xc, ldx, lc, s); break;
        default: return hipErrorInvalidValue;
      }
    }
  }
  if (router) {
    L = logits;
    ldl = E + 1;
  }
  hipLaunchKernelGGL(k_topk, dim3((B + 3) / 4), dim3(256), 0, s, L, ldl, E, B, k,
                     (router && shg) ? 1 : 0, ids, weights, shared_w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// per-expert row lists, rebuilt in LDS by every routed expert workgroup
// ---------------------------------------------------------------------------
struct GatherLds {
  __align__(16) uint32_t key[kMaxPairs];   // expert << 8 | pair, ~0 if unused
  uint32_t skey[kMaxPairs];                // the valid keys in ascending order
  int unique[kMaxPairs];                   // sorted unique experts
  int offsets[kMaxPairs + 1];
  int pairs[kMaxPairs];                    // b*k + j grouped by expert, then b, then j
  int U;
};

// Sorting the keys (expert << 8 | pair index) ascending gives the pairs
// grouped by expert, then by pair index (b, then j).  Each pair's rank is
// the number of smaller keys: the key range is split over PARTS thread
// groups (every thread of a group reads its part of the keys: LDS
// broadcast), whose counts are then added.  In sorted order an expert's
// first pair starts a group, and the groups are numbered by a ballot prefix
// count.  Ids outside [0, E) take no part.  MAXP (compile time) bounds Bk;
// NT = blockDim.x >= MAXP.  Contains __syncthreads: call from uniform
// control flow.
template <int MAXP, int NT>
__device__ void build_gather(const int32_t *__restrict__ ids, int Bk, int E, GatherLds &g) {
  static_assert(MAXP % 4 == 0 && MAXP <= kMaxPairs && MAXP <= 128, "pairs per lane");
  static_assert(NT >= MAXP && NT % 64 == 0, "threads");
  // key groups scanned in parallel (MAXP is a multiple of 16)
  constexpr int PARTS = NT / MAXP >= 4 ? 4 : (NT / MAXP >= 2 ? 2 : 1);
  constexpr int PK = MAXP / PARTS;  // keys per group
  static_assert(MAXP % 16 == 0 && PK % 4 == 0, "keys per group");
  __shared__ int s_rank[PARTS][MAXP], s_nv[PARTS][MAXP];
  const int t = threadIdx.x;
  if (t < MAXP) {
    uint32_t key = 0xFFFFFFFFu;
    if (t < Bk) {
      const int e = ids[t];
      if (e >= 0 && e < E) key = ((uint32_t)e << 8) | (uint32_t)t;
    }
    g.key[t] = key;
  }
  __syncthreads();
  if (t < PARTS * MAXP) {
    const int mi = t % MAXP, part = t / MAXP;
    const uint32_t mine = g.key[mi];
    int rank = 0, nv = 0;
#pragma unroll
    for (int c = 0; c < PK / 4; ++c) {
      const uint4 q = reinterpret_cast<const uint4 *>(g.key)[part * (PK / 4) + c];
      rank += (q.x < mine) + (q.y < mine) + (q.z < mine) + (q.w < mine);
      nv += (q.x != 0xFFFFFFFFu) + (q.y != 0xFFFFFFFFu) + (q.z != 0xFFFFFFFFu) +
            (q.w != 0xFFFFFFFFu);
    }
    s_rank[part][mi] = rank;
    s_nv[part][mi] = nv;
  }
  __syncthreads();
  int nv = 0;  // valid pairs (every thread of the first wave adds the groups)
  if (t < MAXP) {
    const uint32_t mine = g.key[t];
    int rank = 0;
#pragma unroll
    for (int part = 0; part < PARTS; ++part) {
      rank += s_rank[part][t];
      nv += s_nv[part][t];
    }
    if (mine != 0xFFFFFFFFu) g.skey[rank] = mine;
  }
  __syncthreads();
  if (t < 64) {
    int base = 0;
#pragma unroll
    for (int h = 0; h < (MAXP + 63) / 64; ++h) {
      const int r = t + 64 * h;
      const bool valid = r < nv;
      const uint32_t sk = valid ? g.skey[r] : 0u;
      const uint32_t prev = (valid && r > 0) ? g.skey[r - 1] : 0xFFFFFFFFu;
      const bool first = valid && (sk >> 8) != (prev >> 8);
      const unsigned long long bal = __ballot(first);
      const int urank = base + __popcll(bal & ((1ull << t) - 1ull));
      if (valid) g.pairs[r] = (int)(sk & 0xFFu);
      if (first) {
        g.unique[urank] = (int)(sk >> 8);
        g.offsets[urank] = r;
      }
      base += __popcll(bal);
    }
    if (t == 0) {
      g.U = base;
      g.offsets[base] = nv;
    }
  }
  __syncthreads();
}

// Workspace views: Q8_1 of h for P pairs (planar), then per block the
// internal {fp32 d, integer code sum} record; the gather lists K2 publishes
// for K3 (U, unique[Bk], offsets[Bk+1], pairs[Bk]) follow in their region.
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
struct HqView {
  uint8_t *codes;    // [P][I]
  uint16_t *ds;      // [P][I/32][2]  fp16 {d, s}
  i32x2 *dq;         // [P][I/32]     {fp32 bits of d, sum of codes}
};
__device__ inline HqView hq_view(uint8_t *base, int P, int I) {
  HqView v;
  v.codes = base;
  v.ds = reinterpret_cast<uint16_t *>(base + (size_t)P * I);
  v.dq = reinterpret_cast<i32x2 *>(base + (size_t)P * I + (size_t)4 * P * (I / 32));
  return v;
}

struct MoeArgs {
  mmv_moe_layer L;
  const float *X;
  int64_t ldx;
  const int32_t *ids;
  const float *weights;
  const float *shared_w;
  float *Y;
  int64_t ldy;
  uint8_t *hq;
  int32_t *gather;   // published row lists (workspace)
  int P;             // pairs: B*k (+ B with a shared expert)
  int routed_shared; // 1: K2 also runs the shared expert's gate/up tiles
  mmv_moe_debug dbg;
  int has_dbg;
  // fused routing (K1)
  float *logits;     // B x (E+1)
  int gather_ready;  // 1: a previous kernel published the row lists (K2 reads them)
  int32_t *ids_out;
  float *weights_out;
  float *shared_w_out;
  int router_wgs;
  int topk_in_k2;    // 1: every K2 workgroup runs top-k on the logits itself
  float *dpart;      // P x H per-pair down products (the by-expert down path)
  int nrows;         // B (the kernels for more than 8 rows take it at run time)
  int32_t *work;     // B > 8: [0] count, then (slot << 4 | row group) gate/up items
};

// expert e's gate and up planes (strides resolved on the host)
__device__ __forceinline__ void expert_gate_up(const mmv_moe_layer &L, int e, const uint8_t *&gq,
                                               const uint16_t *&gd, const uint8_t *&uq,
                                               const uint16_t *&ud) {
  gq = L.gate_qs + e * L.gate_qs_stride;
  gd = L.gate_d + e * L.gate_d_stride;
  uq = L.up_qs + e * L.up_qs_stride;
  ud = L.up_d + e * L.up_d_stride;
}

// Published row lists (workspace): [0] U, [1, 1+Bk) unique experts,
// [1+Bk, 2+2Bk) offsets, [2+2Bk, 2+3Bk) pairs.  Thread t of a 256-thread
// workgroup holds entries t and t + 256 (gl_n = 3 Bk + 2 <= 386).
__device__ __forceinline__ void put_gather_entry(int idx, int val, int Bk, GatherLds &g) {
  if (idx == 0) g.U = val;
  else if (idx < 1 + Bk) g.unique[idx - 1] = val;
  else if (idx < 2 + 2 * Bk) g.offsets[idx - 1 - Bk] = val;
  else if (idx < 2 + 3 * Bk) g.pairs[idx - 2 - 2 * Bk] = val;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// one gate/up tile: 32 rows of gate and of up, for nr activation rows
// ---------------------------------------------------------------------------
// 4 waves; wave w owns rows 8w..8w+7 of the tile in gate and in up; 16 lanes
// per row, 4 rows per pass; passes: gate rows 0-3, 4-7, up rows 0-3, 4-7, so
// gate row n and up row n land in the same lane group.  T = H / 512 blocks per
// lane per row (compile time: all 4*T weight loads issued before x is
// staged), or 0 for a runtime loop over any H % 32 == 0.
// rowmap / pairmap (LDS) must be written before the call; the call begins
// with the barrier that publishes them.  PRE > 0: the caller already loaded
// the activations of all B rows into xall (PRE float4 tasks per thread,
// issued before routing); they are quantized into stage rows 0..B-1 and
// row r of the tile reads stage row rowmap[r].  PRE == 0: the nr rows
// rowmap[0..nr) are loaded here, into stage rows 0..nr-1.
// mid() runs once the weight loads are in flight, before the activations
// are staged (uniform control flow; it may contain barriers).
template <int B, int T, int PRE, bool SC, int NW, typename Mid>
__device__ __forceinline__ void gate_up_tile(const MoeArgs &a, const uint8_t *gq,
                                             const uint16_t *gd, const uint8_t *uq,
                                             const uint16_t *ud, int tile, int nr,
                                             const int *rowmap, const int *pairmap,
                                             uint8_t *smem, float (*hbuf)[32],
                                             const XPre<(PRE > 0 ? PRE : 1)> &xall, Mid &&mid) {
  const int H = a.L.hidden, I = a.L.inter, nbh = H >> 5, ntiles = I >> 5;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int sub = lane & 15, q = lane >> 4;
  // NW waves share the tile's 32 rows: RPW rows of each matrix per wave, in
  // NG groups of 4 (one row per 16-lane group); p < NG gate, p >= NG up
  constexpr int NT = 64 * NW, RPW = 32 / NW, NG = RPW / 4, NP = 2 * NG;
  static_assert(NW == 4 || (NW == 8 && PRE == 0 && !SC), "8 waves: no preloaded x, no chunked scales");
  int64_t rowoff[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) rowoff[p] = (int64_t)(tile * 32 + RPW * wv + 4 * (p % NG) + q) * nbh;

  constexpr int TT = T > 0 ? T : 1;
  // activations first (loads complete in issue order), then the weights
  // tasks of 4 values: nr * H / 4 <= B * 128 * T over NT threads
  constexpr int MAXT = (T > 0 && PRE == 0) ? cmax(1, cmin(B, 2) * T * 128 / NT) : 1;  // <= 2 rows
  XPre<MAXT> xp;
  __syncthreads();  // rowmap / pairmap visible
  if constexpr (T > 0 && PRE == 0) xpre_load(a.X, a.ldx, rowmap, nr, H, xp, 0, NT);
  // SC (T > 0, 16-byte aligned scale planes): a wave's 8 gate rows and 8 up
  // rows hold 2 x 8 x 32T bytes of fp16 scales, fetched as 16-byte chunks
  // (2T per row) by SCL loads per lane instead of one 2-byte load per (row,
  // block): a load instruction costs issue time whatever its width, and
  // with one workgroup per CU the weights' issue is on the critical path
  // (traced: 1.65 -> 1.0 us without the 2-byte loads).  The chunks go to this
  // wave's LDS rows while the weights are in flight.
  static_assert(!SC || T > 0, "chunked scales need compile-time T");
  constexpr int SCH = 16 * TT;              // chunks per matrix and wave
  constexpr int SCL = (2 * SCH + 63) / 64;  // chunk loads per lane
  __shared__ __align__(16) uint16_t s_sc[SC ? 4 : 1][2][8][16 * TT];  // [wave][gate, up][row][block]
  u32x4 scv[SCL];
  if constexpr (SC) {  // requested before the weights (loads complete in order)
#pragma unroll
    for (int i = 0; i < SCL; ++i) {
      const int c = min(lane + 64 * i, 2 * SCH - 1);
      const int m = c >= SCH ? 1 : 0, cc = c - m * SCH;
      const int rl = cc / (2 * TT), part = cc - rl * 2 * TT;
      scv[i] = load_stream16((m ? ud : gd) + (int64_t)(tile * 32 + 8 * wv + rl) * nbh + 8 * part);
    }
  }
  u32x4 w[NP][TT];
  float dw[NP][TT];
  if constexpr (T > 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int j = sub + 16 * t;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint8_t *wq = p < NG ? gq : uq;
        const uint16_t *wd = p < NG ? gd : ud;
        w[p][t] = load_stream16(wq + (rowoff[p] + j) * 16);
        if constexpr (!SC) dw[p][t] = f16_bits_to_f32(load_stream2(wd + rowoff[p] + j));
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every weight load issued before any wait
  MMV_TL(2);
  mid();
  const XStage st = xstage_at(smem, B, H);
  if constexpr (PRE > 0) {
    xpre_quantize(xall, B, H, st, 0, 256);
  } else if constexpr (T > 0) {
    xpre_quantize(xp, nr, H, st, 0, NT);
    // rows past the preloaded ones (B > 2), in passes of MAXT tasks: the
    // weights are in flight meanwhile, so registers are short here
    stage_quantize<MAXT>(a.X, a.ldx, rowmap, nr, H, st, MAXT * NT, NT);
  } else {
    stage_quantize(a.X, a.ldx, rowmap, nr, H, st);
  }
  if constexpr (SC) {  // the scale chunks (in before the weights) to this wave's LDS rows
#pragma unroll
    for (int i = 0; i < SCL; ++i) {
      const int c = lane + 64 * i;
      if (c < 2 * SCH) {
        const int m = c >= SCH ? 1 : 0, cc = c - m * SCH;
        const int rl = cc / (2 * TT), part = cc - rl * 2 * TT;
        *reinterpret_cast<u32x4 *>(&s_sc[wv][m][rl][8 * part]) = scv[i];
      }
    }
  }
  __syncthreads();
  // gate row n and up row n of one activation row -> h (lanes sub == 0)
  auto put_h = [&](int r, const float (&a4)[NP]) {
#pragma unroll
    for (int hh = 0; hh < NG; ++hh) {
      const float gv = row16_sum(a4[hh]);
      const float uv = row16_sum(a4[NG + hh]);
      const float h = silu_f(gv) * uv;
      const int nl = RPW * wv + 4 * hh + q;
      if (sub == 0) {
        hbuf[r][nl] = h;
        if (a.has_dbg) {
          const int64_t o = (int64_t)pairmap[r] * I + tile * 32 + nl;
          if (a.dbg.h) a.dbg.h[o] = h;
          if (a.dbg.gate_out) a.dbg.gate_out[o] = gv;
          if (a.dbg.up_out) a.dbg.up_out[o] = uv;
        }
      }
    }
  };
  {
    int srow[B];  // stage row of tile row r
#pragma unroll
    for (int r = 0; r < B; ++r) srow[r] = PRE > 0 ? rowmap[min(r, nr - 1)] : r;

    float acc[NP][B];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int r = 0; r < B; ++r) acc[p][r] = 0.0f;
    auto block = [&](const u32x4 (&wb)[NP], const float (&db)[NP], int j) {
#pragma unroll
      for (int r = 0; r < B; ++r) {
        if (r < nr) {
          const int sr = srow[r];
          const i32x4 xa = xstage_lo(st, sr, H, j);
          const i32x4 xb = xstage_hi(st, sr, H, j);
          const int xs = st.qsum[sr * nbh + j];
          const float dx = st.d[sr * nbh + j];
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const int Iv = q4_block_isum(wb[p], xa, xb, xs);
            acc[p][r] = fmaf(db[p] * dx, (float)Iv, acc[p][r]);
          }
        }
      }
    };
    if constexpr (T > 0) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        u32x4 wb[NP];
        float db[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          wb[p] = w[p][t];
          if constexpr (SC)
            db[p] = f16_bits_to_f32(s_sc[wv][p >> 1][4 * (p & 1) + q][sub + 16 * t]);
          else
            db[p] = dw[p][t];
        }
        block(wb, db, sub + 16 * t);
      }
    } else {
      for (int j = sub; j < nbh; j += 16) {
        u32x4 wb[NP];
        float db[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const uint8_t *wq = p < NG ? gq : uq;
          const uint16_t *wd = p < NG ? gd : ud;
          wb[p] = load_stream16(wq + (rowoff[p] + j) * 16);
          db[p] = f16_bits_to_f32(load_stream2(wd + rowoff[p] + j));
        }
        block(wb, db, j);
      }
    }
#pragma unroll
    for (int r = 0; r < B; ++r) {
      if (r < nr) {
        float a4[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) a4[p] = acc[p][r];
        put_h(r, a4);
      }
    }
  }
  __syncthreads();
  MMV_TL(3);

  // Q8_1 epilogue: the 32 h values of (row r, tile) are one block
  if (threadIdx.x < (unsigned)(8 * nr)) {
    const int r = threadIdx.x >> 3, s = threadIdx.x & 7;
    const f32x4 v = *reinterpret_cast<const f32x4 *>(&hbuf[r][4 * s]);
    const Q8Block qb = q8_1_quantize8(v);
    const HqView hv = hq_view(a.hq, a.P, I);
    const int p = pairmap[r];
    *reinterpret_cast<uint32_t *>(hv.codes + (size_t)p * I + tile * 32 + 4 * s) = qb.codes;
    if (s == 0) {
      const size_t bi = (size_t)p * ntiles + tile;
      hv.ds[bi * 2 + 0] = qb.d16;
      hv.ds[bi * 2 + 1] = qb.s16;
      hv.dq[bi] = i32x2{(int32_t)__float_as_uint(f16_bits_to_f32(qb.d16)), qb.qsum};
    }
    if (a.has_dbg && a.dbg.h_q8) {  // the same planar layout as the workspace copy
      uint8_t *dq8 = static_cast<uint8_t *>(a.dbg.h_q8);
      *reinterpret_cast<uint32_t *>(dq8 + (size_t)p * I + tile * 32 + 4 * s) = qb.codes;
      if (s == 0) {
        uint16_t *dds = reinterpret_cast<uint16_t *>(dq8 + (size_t)a.P * I);
        const size_t bi = (size_t)p * ntiles + tile;
        dds[bi * 2 + 0] = qb.d16;
        dds[bi * 2 + 1] = qb.s16;
      }
    }
  }
  MMV_TL_END(kTlGateUp, 4);
}

// both scale planes 16-byte aligned (the chunked scale loads)
__device__ __forceinline__ bool scales16(const uint16_t *gd, const uint16_t *ud) {
  return ((reinterpret_cast<uintptr_t>(gd) | reinterpret_cast<uintptr_t>(ud)) & 15) == 0;
}

// ---------------------------------------------------------------------------
// K2: routed gate/up.  grid = (B*k [+1 shared]) slots x (I/32) tiles.
// ---------------------------------------------------------------------------
template <int B, int T, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_moe_gate_up(MoeArgs a) {
  __shared__ GatherLds g;
  __shared__ int rowmap[MMV_MAX_BATCH];
  __shared__ int pairmap[MMV_MAX_BATCH];
  __shared__ float hbuf[MMV_MAX_BATCH][32];
  extern __shared__ __align__(16) uint8_t smem[];

  __shared__ int s_ids[kMaxPairs];
  __shared__ float s_w[kMaxPairs];
  __shared__ float s_sw[MMV_MAX_BATCH];

  const mmv_moe_layer &L = a.L;
  const int k = L.top_k, H = L.hidden, I = L.inter;
  const int Bk = B * k;
  const int ntiles = I >> 5;
  // slot 0 is the shared expert's when K2 runs it (dispatched first: its
  // tiles carry every row), then one slot per routed expert
  const int slot0 = blockIdx.x / ntiles, tile = blockIdx.x - slot0 * ntiles;
  const bool shared_slot = a.routed_shared && slot0 == 0;
  const int slot = slot0 - a.routed_shared;
  MMV_TL(0);

  // B <= 2: the activations of every row are loaded before routing (they do
  // not depend on it) and stay in registers until the weights are in flight
  constexpr int PRE = (B <= 2 && T > 0) ? B * T / 2 : 0;
  XPre<(PRE > 0 ? PRE : 1)> xall;
  if constexpr (PRE > 0) {
    xpre_load(a.X, a.ldx, nullptr, B, H, xall, 0, 256);
    __builtin_amdgcn_sched_barrier(0);
  }

  const int32_t *ids = a.ids;
  const int E = L.n_experts;
  if (a.topk_in_k2) {
    // routing from the logits K1 wrote; block 0 publishes it for K3
    topk_any(a.logits, E + 1, E, B, k, L.shared_gate_row ? 1 : 0, s_ids, s_w, s_sw);
    __syncthreads();
    if (blockIdx.x == 0) {
      const int t = threadIdx.x;
      if (t < Bk) { a.ids_out[t] = s_ids[t]; a.weights_out[t] = s_w[t]; }
      if (t < B) a.shared_w_out[t] = s_sw[t];
    }
    ids = s_ids;
  }
  MMV_TL(1);  // routing known (top-k inside, or the row lists next)
  // row lists for the down kernel (and the debug copies), from block 0
  auto publish_gather = [&]() {
    const int t = threadIdx.x;
    int32_t *gl = a.gather;
    if (t == 0) gl[0] = g.U;
    if (t < g.U) gl[1 + t] = g.unique[t];
    if (t <= g.U) gl[1 + Bk + t] = g.offsets[t];
    if (t < g.offsets[g.U]) gl[2 + 2 * Bk + t] = g.pairs[t];
    if (a.has_dbg) {
      if (a.dbg.unique && t < g.U) a.dbg.unique[t] = g.unique[t];
      if (a.dbg.offsets && t <= g.U) a.dbg.offsets[t] = g.offsets[t];
      if (a.dbg.pairs && t < g.offsets[g.U]) a.dbg.pairs[t] = g.pairs[t];
      if (a.dbg.n_unique && t == 0) a.dbg.n_unique[0] = g.U;
    }
  };

  if constexpr (B == 1) {
    if (a.topk_in_k2) {
      // One row and the ids this kernel selected (valid and distinct): slot
      // j is the j-th selected expert, pair j.  The weights are requested at
      // once; block 0 builds the row lists for the down kernel while its
      // weights are in flight.
      if (!shared_slot && slot >= k) return;  // uniform over the workgroup
      const uint8_t *gq, *uq;
      const uint16_t *gd, *ud;
      if (shared_slot) {
        gq = L.sh_gate_qs; gd = L.sh_gate_d; uq = L.sh_up_qs; ud = L.sh_up_d;
      } else {
        expert_gate_up(L, s_ids[slot], gq, gd, uq, ud);
      }
      if (threadIdx.x == 0) {
        rowmap[0] = 0;
        pairmap[0] = shared_slot ? Bk : slot;
      }
      auto mid = [&]() {
        if (blockIdx.x == 0) {
          build_gather<MMV_MAX_TOPK, 256>(s_ids, Bk, E, g);
          publish_gather();
        }
      };
      if (T > 0 && scales16(gd, ud))  // uniform
        gate_up_tile<B, T, PRE, (T > 0 && B <= 2), 4>(a, gq, gd, uq, ud, tile, 1, rowmap, pairmap, smem,
                                         hbuf, xall, mid);
      else
        gate_up_tile<B, T, PRE, false, 4>(a, gq, gd, uq, ud, tile, 1, rowmap, pairmap, smem, hbuf,
                                       xall, mid);
      return;
    }
  }

  if (a.gather_ready) {  // the top-k kernel published the row lists
    const int t = threadIdx.x, gl_n = 3 * Bk + 2;
    const int g0 = a.gather[min(t, gl_n - 1)], g1 = a.gather[min(t + 256, gl_n - 1)];
    if (t < gl_n) put_gather_entry(t, g0, Bk, g);
    if (t + 256 < gl_n) put_gather_entry(t + 256, g1, Bk, g);
    __syncthreads();
  } else {
    build_gather<cmin(B * MMV_MAX_TOPK, kMaxPairs), 256>(ids, Bk, E, g);
    if (blockIdx.x == 0) publish_gather();
  }
  if (!shared_slot && slot >= g.U) return;  // uniform over the workgroup

  const uint8_t *gq, *uq;
  const uint16_t *gd, *ud;
  int nr;
  if (shared_slot) {
    gq = L.sh_gate_qs; gd = L.sh_gate_d; uq = L.sh_up_qs; ud = L.sh_up_d;
    nr = B;
  } else {
    expert_gate_up(L, g.unique[slot], gq, gd, uq, ud);
    // an expert appears at most once per row when ids are valid (distinct
    // within a row); the clamp keeps duplicated ids memory-safe
    nr = min(g.offsets[slot + 1] - g.offsets[slot], B);
  }
  if (threadIdx.x < (unsigned)nr) {
    const int r = threadIdx.x;
    const int p = shared_slot ? Bk + r : g.pairs[g.offsets[slot] + r];
    pairmap[r] = p;
    rowmap[r] = shared_slot ? r : p / k;
  }
  // chunked scales for one or two rows (at one workgroup per CU the issue
  // time counts); more rows keep more workgroups per CU, and there the
  // extra registers cost more than the issue time saved (B = 8: +0.3 us)
  if (T > 0 && B <= 2 && scales16(gd, ud))  // uniform
    gate_up_tile<B, T, PRE, (T > 0 && B <= 2), NW>(a, gq, gd, uq, ud, tile, nr, rowmap, pairmap, smem, hbuf,
                                     xall, []() {});
  else
    gate_up_tile<B, T, PRE, false, NW>(a, gq, gd, uq, ud, tile, nr, rowmap, pairmap, smem, hbuf,
                                   xall, []() {});
}

// ---------------------------------------------------------------------------
// K1: router rows (one wave per row, logits to the workspace)
// ---------------------------------------------------------------------------
template <int B, int HC>
__global__ __launch_bounds__(256) void k_moe_router(MoeArgs a) {
  const mmv_moe_layer &L = a.L;
  const int E = L.n_experts, H = L.hidden;
  const int e = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  MMV_TL(0);
  if (e < E + (L.shared_gate_row ? 1 : 0)) {
    const float *row = e < E ? L.router + (int64_t)e * H : L.shared_gate_row;
    router_row<B, HC>(row, H, a.X, a.ldx, a.logits + e, E + 1);
  }
  MMV_TL_END(kTlRouter, 1);
}

// ---------------------------------------------------------------------------
// K1b (more rows): one workgroup, a wave per row, runs top-k for every
// row, builds the row lists and publishes both, so the gate/up workgroups
// only read them.
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(512) void k_moe_topk_gather(MoeArgs a) {
  __shared__ GatherLds g;
  __shared__ int s_ids[kMaxPairs];
  __shared__ float s_w[kMaxPairs];
  __shared__ float s_sw[MMV_MAX_BATCH];
  const mmv_moe_layer &L = a.L;
  const int E = L.n_experts, k = L.top_k, Bk = B * k, t = threadIdx.x;
  MMV_TL(0);
  topk_any(a.logits, E + 1, E, B, k, L.shared_gate_row ? 1 : 0, s_ids, s_w, s_sw);
  __syncthreads();
  MMV_TL(1);
  if (t < Bk) { a.ids_out[t] = s_ids[t]; a.weights_out[t] = s_w[t]; }
  if (t < B) a.shared_w_out[t] = s_sw[t];
  build_gather<cmin(B * MMV_MAX_TOPK, kMaxPairs), 64 * B>(s_ids, Bk, E, g);
  int32_t *gl = a.gather;
  if (t == 0) gl[0] = g.U;
  if (t < g.U) gl[1 + t] = g.unique[t];
  if (t <= g.U) gl[1 + Bk + t] = g.offsets[t];
  if (t < g.offsets[g.U]) gl[2 + 2 * Bk + t] = g.pairs[t];
  MMV_TL_END(kTlTopkGather, 2);
}

// ---------------------------------------------------------------------------
// K3: down + weighted combine + shared expert (one kernel)
// ---------------------------------------------------------------------------
// NWV waves (8 for B = 3, 4; else 4); the workgroup owns 4 output rows (lane
// group q of every wave = row 4*blockIdx + q).  Wave w takes the experts with
// id % NWV == w, wave 0 also the shared expert last; each (row, pair)
// product goes to LDS, and after the expert loop a row's pairs are added
// by the slot tree (down_combine_tree), so which wave held an expert does
// not change any bit.  Q8_1(h) of every pair is staged in LDS (codes, fp32
// d, integer sums).  Order of work, so that no wait covers more than it
// needs (loads complete in issue order): the row lists are requested and go
// to LDS, and each wave's expert list is built; the wave's first chunk of
// expert weights is requested, then Q8_1(h) goes straight into LDS.  The
// first chunk covers every expert of the wave for typical batches (one load
// latency for all of them); experts beyond it follow in double-buffered
// chunks of kDownCH (the next requested before the current one is used).
// Loads within a chunk are unconditional: a slot past the end of the
// wave's list re-reads its last expert (or expert 0 for an empty list) and
// is not used.  TI = I / 512 (compile time) or 0 (runtime loop over
// I % 32 == 0, one block at a time).
constexpr int kDownCH = 4;  // experts per weight chunk after the first

// one (pair, block) term of a down product: d_w d_h sum_i (q_i - 8) c_i
__device__ __forceinline__ float down_block_value(u32x4 wb, float db, i32x4 xa, i32x4 xb,
                                                  float dx, int qs) {
  return (db * dx) * (float)q4_block_isum(wb, xa, xb, qs);
}

// The sum over a row's slots: the pairwise tree row16_sum forms over 16
// lanes (lane j = slot j, zero past k), written out for one thread; float
// addition commutes, so every lane of the DPP tree and this code agree.
__device__ __forceinline__ float down_combine_tree(const float (&p)[16]) {
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = (p[4 * i] + p[4 * i + 1]) + (p[4 * i + 2] + p[4 * i + 3]);
  return (q[0] + q[1]) + (q[2] + q[3]);
}

// Scales stay fp16 bits until the products: converted where they are
// loaded, they make the compiler wait for the weight loads before anything
// requested after them (Q8_1(h)).
template <int TI, int CH = kDownCH>
struct DownChunk {
  static constexpr int kCH = CH;
  u32x4 w[CH][TI > 0 ? TI : 1];
  uint16_t d[CH][TI > 0 ? TI : 1];
};


// experts in a wave's first chunk: every expert of the wave for typical
// batches (experts are split over the 4 waves by id % 4, so about U / 4 each;
// B = 8 at E = 512, k = 10 has U ~ 75), so their loads are in flight together
// instead of one chunk latency after another
template <int B>
constexpr int down_first_chunk() { return B == 1 ? 4 : (B == 2 ? 8 : 4); }

template <int B, int TI, int NWV>
__global__ __launch_bounds__(64 * NWV) void k_moe_down(MoeArgs a) {
  __shared__ int s_unique[kMaxPairs];
  __shared__ int s_off[kMaxPairs + 1];
  __shared__ int s_pairs[kMaxPairs];
  __shared__ int s_prow[kMaxPairs];  // activation row of s_pairs[i]
  __shared__ int s_wl[NWV][kMaxPairs + 1];
  __shared__ int s_wn[NWV];
  __shared__ int s_U;
  __shared__ float s_pw[kMaxPairs + MMV_MAX_BATCH];
  __shared__ float s_dot[4][kMaxPairs + MMV_MAX_BATCH];  // per output row, per pair
  extern __shared__ __align__(16) uint8_t smem[];

  const mmv_moe_layer &L = a.L;
  const int k = L.top_k, H = L.hidden, I = L.inter;
  const int Bk = B * k, P = a.P, nbi = I >> 5;
  const bool has_sh = L.sh_down_qs != nullptr;
  const int t = threadIdx.x;

  MMV_TL(0);
  // ---- prologue loads: row lists and pair weights
  const int gl_n = 3 * Bk + 2;
  const int g0 = a.gather[min(t, gl_n - 1)];
  const int g1 = a.gather[min(t + 256, gl_n - 1)];
  const int pwi = min(t, Bk + B - 1);
  const float pwv = pwi < Bk ? a.weights[pwi] : (a.shared_w ? a.shared_w[pwi - Bk] : 1.0f);
  const HqView hv = hq_view(a.hq, P, I);
  const int n16 = P * I / 16, nblk = P * nbi;

  // ---- row lists to LDS, per-wave expert lists
  // gather region: [0] U, [1, 1+Bk) unique, [1+Bk, 2+2Bk) offsets, [2+2Bk, 2+3Bk) pairs
  auto put_gather = [&](int idx, int val) {
    if (idx == 0) s_U = val;
    else if (idx < 1 + Bk) s_unique[idx - 1] = val;
    else if (idx >= 1 + Bk && idx < 2 + 2 * Bk) s_off[idx - 1 - Bk] = val;
    else if (idx >= 2 + 2 * Bk && idx < gl_n) {
      s_pairs[idx - 2 - 2 * Bk] = val;
      s_prow[idx - 2 - 2 * Bk] = val / k;
    }
  };
  put_gather(t, g0);
  put_gather(t + 256, g1);
  if (t < Bk + B) s_pw[t] = pwv;
  // pairs that no expert list holds (ids outside [0, E)) add zero
  for (int i = t; i < 4 * (kMaxPairs + MMV_MAX_BATCH); i += 64 * NWV) (&s_dot[0][0])[i] = 0.0f;
  __syncthreads();
  MMV_TL(1);  // row lists in LDS
  const int U = s_U;
  // per-wave expert lists: class = id % NWV, ascending; shared expert (index
  // U) appended to wave 0
  if (t < 64) {  // wave 0: list positions by ballot prefix counts
    int base[NWV];
#pragma unroll
    for (int c = 0; c < NWV; ++c) base[c] = 0;
    const unsigned long long lt = (1ull << t) - 1ull;
#pragma unroll
    for (int h = 0; h < kMaxPairs / 64; ++h) {
      const int u = t + 64 * h;
      const int cls = u < U ? (s_unique[u] % NWV) : -1;
#pragma unroll
      for (int c = 0; c < NWV; ++c) {
        const unsigned long long bal = __ballot(cls == c);
        if (cls == c) s_wl[c][base[c] + __popcll(bal & lt)] = u;
        base[c] += __popcll(bal);
      }
    }
    if (t == 0) {
      if (has_sh) s_wl[0][base[0]++] = U;
#pragma unroll
      for (int c = 0; c < NWV; ++c) s_wn[c] = base[c];
    }
  }
  __syncthreads();

  const int lane = t & 63, wv = t >> 6, sub = lane & 15, q = lane >> 4;
  const int row = blockIdx.x * 4 + q;
  const int rowc = min(row, H - 1);
  const int n = s_wn[wv];
  const int *wl = s_wl[wv];

  // list entry c of this wave -> weight planes of its expert (expert 0 for
  // an empty list: a valid address whose data is never used)
  auto expert_ptr = [&](int c, const uint8_t *&dq, const uint16_t *&dd) {
    const int u = n > 0 ? wl[min(c, n - 1)] : -1;
    if (u >= 0 && u < U) {
      dq = L.down_qs + s_unique[u] * L.down_qs_stride;
      dd = L.down_d + s_unique[u] * L.down_d_stride;
    } else if (u == U) {
      dq = L.sh_down_qs; dd = L.sh_down_d;
    } else {
      dq = L.down_qs; dd = L.down_d;
    }
  };
  auto load_chunk = [&](int c0, auto &ch) {
    constexpr int CH = std::remove_reference_t<decltype(ch)>::kCH;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint8_t *dq;
      const uint16_t *dd;
      expert_ptr(c0 + c, dq, dd);
#pragma unroll
      for (int ti = 0; ti < TI; ++ti) {
        const int64_t blk = (int64_t)rowc * nbi + sub + 16 * ti;
        ch.w[c][ti] = load_stream16(dq + blk * 16);
        ch.d[c][ti] = load_stream2(dd + blk);
      }
    }
  };

  constexpr int NF = down_first_chunk<B>();
  DownChunk<TI, NF> first;
  DownChunk<TI> cha, chb;
  if constexpr (TI > 0) {
    load_chunk(0, first);
    if (n > NF) load_chunk(NF, cha);  // uniform over the wave
  }
  __builtin_amdgcn_sched_barrier(0);
  MMV_TL(2);

  // ---- Q8_1(h) from global memory straight into LDS (global_load_lds: a
  // wave instruction fills 64 consecutive 16- or 4-byte LDS slots, lane l
  // the l-th), requested after the weights: it is needed only once they
  // have arrived, and it occupies no registers.  Codes go to the half-plane
  // layout: LDS chunk o of a row holds source chunk 2 (o % nbi) + o / nbi.
  const XStage hs = xstage_at(smem, P, I);
  {
    const int ln = t & 63, wq = t >> 6;
    for (int m = wq; 64 * m < n16; m += NWV) {
      const int dc = 64 * m + ln;
      if (dc < n16) {
        const int r = dc / (2 * nbi), o = dc - r * 2 * nbi;
        const int half = o >= nbi ? 1 : 0;
        const int sc = r * 2 * nbi + 2 * (o - half * nbi) + half;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(hv.codes + 16 * (size_t)sc),
            (__attribute__((address_space(3))) void *)(hs.codes + 1024 * m), 16, 0, 0);
      }
    }
    for (int m = wq; 64 * m < nblk; m += NWV) {
      const int bi = 64 * m + ln;
      if (bi < nblk) {
        const uint8_t *src = reinterpret_cast<const uint8_t *>(hv.dq + bi);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(hs.d + 64 * m),
                                         4, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(src + 4),
            (__attribute__((address_space(3))) void *)(hs.qsum + 64 * m), 4, 0, 0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS writes done; the barrier publishes them
  __syncthreads();
  MMV_TL(3);  // Q8_1(h) staged

  // Each pair's product with its expert is formed whole, in one order for
  // every B and whichever wave holds the expert: per lane the blocks it owns
  // (ascending), then the 16-lane sum; a row's pairs are added after the
  // expert loop by a fixed tree over its slots, as k_moe_combine adds them.
  struct PairData {
    i32x4 xa, xb;
    int qs;
    float dx;
  };
  auto pair_load = [&](int p, int j, PairData &pd) {
    pd.xa = xstage_lo(hs, p, I, j);
    pd.xb = xstage_hi(hs, p, I, j);
    pd.qs = hs.qsum[p * nbi + j];
    pd.dx = hs.d[p * nbi + j];
  };
  auto pair_value = [&](const PairData &pd, const u32x4 wb, const float db) {
    return down_block_value(wb, db, pd.xa, pd.xb, pd.dx, pd.qs);
  };
  auto put_dot = [&](int p, float v) {
    v = row16_sum(v);
    if (sub == 0) s_dot[q][p] = v;
  };
  // every pair of list entries c0 .. c0 + CH - 1.  In groups of 4 experts,
  // the list metadata, then the first pair's LDS data of each expert are
  // read together (independent reads in flight), so most experts (one pair
  // each when rows share few experts) cost no dependent LDS round trip of
  // their own, and their 16-lane sums run interleaved.
  auto consume_chunk = [&](const auto &ch, int c0) {
    constexpr int CH = std::remove_reference_t<decltype(ch)>::kCH;
    constexpr int MG = cmin(CH, 4);
#pragma unroll
    for (int c4 = 0; c4 < CH; c4 += MG) {
      int pbeg[MG], pend[MG], isu[MG], p0[MG];
      bool val[MG];
#pragma unroll
      for (int c = 0; c < MG; ++c) {
        const int u = wl[min(c0 + c4 + c, max(n - 1, 0))];
        val[c] = c0 + c4 + c < n;
        isu[c] = u < U;
        pbeg[c] = isu[c] ? s_off[u] : 0;
        pend[c] = isu[c] ? min(s_off[u + 1], s_off[u] + B) : B;
      }
#pragma unroll
      for (int c = 0; c < MG; ++c) p0[c] = isu[c] ? s_pairs[pbeg[c]] : Bk;
      PairData pd[MG][TI];
#pragma unroll
      for (int c = 0; c < MG; ++c)
#pragma unroll
        for (int ti = 0; ti < TI; ++ti) pair_load(p0[c], sub + 16 * ti, pd[c][ti]);
      float v0[MG];
#pragma unroll
      for (int c = 0; c < MG; ++c) {
        v0[c] = 0.0f;
#pragma unroll
        for (int ti = 0; ti < TI; ++ti)
          v0[c] += pair_value(pd[c][ti], ch.w[c4 + c][ti], f16_bits_to_f32(ch.d[c4 + c][ti]));
      }
      gsum_last_n<16, MG>(v0);  // the same sums as row16_sum, interleaved
#pragma unroll
      for (int c = 0; c < MG; ++c)
        if (val[c] && sub == 0) s_dot[q][p0[c]] = v0[c];
#pragma unroll
      for (int c = 0; c < MG; ++c) {
        if (val[c]) {
          for (int pi = pbeg[c] + 1; pi < pend[c]; ++pi) {
            const int p = isu[c] ? s_pairs[pi] : Bk + pi;
            float v = 0.0f;
#pragma unroll
            for (int ti = 0; ti < TI; ++ti) {
              PairData pdx;
              pair_load(p, sub + 16 * ti, pdx);
              v += pair_value(pdx, ch.w[c4 + c][ti], f16_bits_to_f32(ch.d[c4 + c][ti]));
            }
            put_dot(p, v);
          }
        }
      }
    }
  };

  if constexpr (TI > 0) {
    consume_chunk(first, 0);
    // beyond the first chunk (rare): double-buffered chunks of kDownCH
    for (int c0 = NF; c0 < n; c0 += 2 * kDownCH) {
      load_chunk(c0 + kDownCH, chb);  // re-reads the last expert past the end
      consume_chunk(cha, c0);
      if (c0 + 2 * kDownCH < n) load_chunk(c0 + 2 * kDownCH, cha);
      if (c0 + kDownCH < n) consume_chunk(chb, c0 + kDownCH);
    }
  } else {
    for (int c = 0; c < n; ++c) {
      const uint8_t *dq;
      const uint16_t *dd;
      expert_ptr(c, dq, dd);
      const int u = wl[c];
      const bool su = u < U;
      const int pb0 = su ? s_off[u] : 0;
      const int np = su ? min(s_off[u + 1] - pb0, B) : B;
      float vp[B];
#pragma unroll
      for (int r = 0; r < B; ++r) vp[r] = 0.0f;
      for (int j = sub; j < nbi; j += 16) {
        const int64_t blk = (int64_t)rowc * nbi + j;
        const u32x4 wb = load_stream16(dq + blk * 16);
        const float db = f16_bits_to_f32(load_stream2(dd + blk));
#pragma unroll
        for (int r = 0; r < B; ++r) {
          if (r < np) {
            PairData pd;
            pair_load(su ? s_pairs[pb0 + r] : Bk + r, j, pd);
            vp[r] += pair_value(pd, wb, db);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < B; ++r)
        if (r < np) put_dot(su ? s_pairs[pb0 + r] : Bk + r, vp[r]);
    }
  }

  __syncthreads();
  if (a.has_dbg && a.dbg.down_out) {  // each (output row, pair) product, unweighted
    for (int i = t; i < 4 * P; i += 64 * NWV) {
      const int qq = i / P, p = i - qq * P, r = blockIdx.x * 4 + qq;
      if (r < H) a.dbg.down_out[(int64_t)p * H + r] = s_dot[qq][p];
    }
  }
  // each row's pairs: lane j of a 16-lane group takes slot j (zero past k),
  // the products w * dot summed by the 16-lane tree, then the shared term
  // (down_combine_tree is the same sum, written out)
  for (int b = wv; b < B; b += NWV) {  // uniform over the wave
    const int j = sub;
    const int p = b * k + min(j, k - 1);
    const float prod = j < k ? s_pw[p] * s_dot[q][p] : 0.0f;
    float v = row16_sum(prod);
    if (has_sh) v = fmaf(s_pw[Bk + b], s_dot[q][Bk + b], v);
    const int r = blockIdx.x * 4 + q;
    if (sub == 0 && r < H) a.Y[(int64_t)b * a.ldy + r] = v;
  }
  MMV_TL_END(kTlDown, 4);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// K3 by expert (more rows) + combine
// ---------------------------------------------------------------------------
// With many rows the one-kernel down projection walks every unique expert
// in every output-row workgroup and stages Q8_1(h) of all pairs in each of
// them.  Here a workgroup owns one expert slot (the shared expert first,
// then the unique routed experts) and 64 output rows: it reads that
// 64 x I block of the expert's Down once, Q8_1(h) of the slot's pairs
// straight from the workspace (at most 4 pairs in flight), and writes each
// pair's product to the workspace (dpart[p * H + n]), formed as in K3
// (per lane its blocks ascending, then the 16-lane sum), so the result is
// the same bit for bit.  k_moe_combine then adds each row's pairs in slot
// order.  A slot's expert and pair range come from the published row lists;
// slots past the number of unique experts exit.
constexpr int kDownPartRows = 64;

template <int B, int TI>  // B = 0: rows at run time (a.nrows <= 64)
__global__ __launch_bounds__(256) void k_moe_down_part(MoeArgs a) {
  constexpr int RP = kDownPartRows / 16;             // rows per 16-lane group
  constexpr int NP = (B > 0 && B < 4) ? B : 4;       // pairs whose Q8_1(h) is in flight together
  constexpr int TT = TI > 0 ? TI : 1;
  const mmv_moe_layer &L = a.L;
  const int Bv = B > 0 ? B : a.nrows;
  const int k = L.top_k, H = L.hidden, I = L.inter;
  const int Bk = Bv * k, nbi = I >> 5;
  const int has_sh = L.sh_down_qs != nullptr ? 1 : 0;
  const int ntile = (H + kDownPartRows - 1) / kDownPartRows;
  const int slot0 = blockIdx.x / ntile, tile = blockIdx.x - slot0 * ntile;
  const bool shared_slot = has_sh && slot0 == 0;
  const int u = slot0 - has_sh;  // < Bk: every list entry read below is in bounds
  const int32_t *gl = a.gather;
  MMV_TL(0);
  const uint8_t *dq;
  const uint16_t *dd;
  int np, pbase;
  if (shared_slot) {
    dq = L.sh_down_qs; dd = L.sh_down_d;
    np = Bv; pbase = 0;
  } else {
    const int U = gl[0], e = gl[1 + u], o0 = gl[1 + Bk + u], o1 = gl[2 + Bk + u];
    if (u >= U) return;  // uniform over the workgroup
    dq = L.down_qs + e * L.down_qs_stride;
    dd = L.down_d + e * L.down_d_stride;
    np = min(o1 - o0, Bv);  // a row meets an expert once: at most one pair per row
    pbase = o0;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, sub = lane & 15, q = lane >> 4;
  const int row0 = tile * kDownPartRows + 16 * wv + q;  // + 4 rp
  // the slot's pair indices, lane r holding the r-th, requested before the
  // weights (loads complete in issue order: waiting for these does not wait
  // for the weights)
  const int pl_r = gl[2 + 2 * Bk + pbase + min(lane, max(np - 1, 0))];
  const int pl = shared_slot ? Bk + min(lane, Bv - 1) : pl_r;
  u32x4 w[RP][TT];
  uint16_t dw[RP][TT];  // fp16 bits until use (see DownChunk)
  if constexpr (TI > 0) {
#pragma unroll
    for (int rp = 0; rp < RP; ++rp) {
      const int rowc = min(row0 + 4 * rp, H - 1);
#pragma unroll
      for (int ti = 0; ti < TI; ++ti) {
        const int64_t blk = (int64_t)rowc * nbi + sub + 16 * ti;
        w[rp][ti] = load_stream16(dq + blk * 16);
        dw[rp][ti] = load_stream2(dd + blk);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  MMV_TL(1);
  const HqView hv = hq_view(a.hq, a.P, I);
  auto store_dots = [&](int p, float (&v)[RP]) {
    gsum_last_n<16, RP>(v);  // the same sums as row16_sum, interleaved
    if (sub == 0) {
#pragma unroll
      for (int rp = 0; rp < RP; ++rp)
        if (row0 + 4 * rp < H) a.dpart[(int64_t)p * H + row0 + 4 * rp] = v[rp];
    }
  };
  // NP pairs at a time: the Q8_1(h) loads of the group, then its products.
  // The first group is straight-line code, so that nothing working on the
  // weights (scale conversion, nibble masks) is hoisted above its loads;
  // more groups (the shared expert for B > 4, or an expert that more than 4
  // rows chose) follow in a loop.
  auto pair_group = [&](int r0) {
    int pp[NP];
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      pp[c] = __builtin_amdgcn_readlane(pl, min(r0 + c, np - 1));
    }
    if constexpr (TI > 0) {
      i32x4 xa[NP][TT], xb[NP][TT];
      int xd[NP][TT], xs[NP][TT];
#pragma unroll
      for (int c = 0; c < NP; ++c)
#pragma unroll
        for (int ti = 0; ti < TI; ++ti) {
          const int j = sub + 16 * ti;
          const int8_t *cb = reinterpret_cast<const int8_t *>(hv.codes) + (size_t)pp[c] * I + 32 * j;
          xa[c][ti] = *reinterpret_cast<const i32x4 *>(cb);
          xb[c][ti] = *reinterpret_cast<const i32x4 *>(cb + 16);
          const int *rec = reinterpret_cast<const int *>(hv.dq + (size_t)pp[c] * nbi + j);
          xd[c][ti] = rec[0];
          xs[c][ti] = rec[1];
        }
      __builtin_amdgcn_sched_barrier(0);  // the loads above go out before any product
#pragma unroll
      for (int c = 0; c < NP; ++c) {
        if (r0 + c < np) {  // uniform
          float v[RP];
#pragma unroll
          for (int rp = 0; rp < RP; ++rp) {
            v[rp] = 0.0f;
#pragma unroll
            for (int ti = 0; ti < TI; ++ti) {
              v[rp] += down_block_value(w[rp][ti], f16_bits_to_f32(dw[rp][ti]), xa[c][ti],
                                        xb[c][ti], __int_as_float(xd[c][ti]), xs[c][ti]);
            }
          }
          store_dots(pp[c], v);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NP; ++c) {
        if (r0 + c < np) {  // uniform
          float v[RP];
#pragma unroll
          for (int rp = 0; rp < RP; ++rp) v[rp] = 0.0f;
          for (int j = sub; j < nbi; j += 16) {
            const int8_t *cb = reinterpret_cast<const int8_t *>(hv.codes) + (size_t)pp[c] * I + 32 * j;
            const i32x4 xa = *reinterpret_cast<const i32x4 *>(cb);
            const i32x4 xb = *reinterpret_cast<const i32x4 *>(cb + 16);
            const int *rec = reinterpret_cast<const int *>(hv.dq + (size_t)pp[c] * nbi + j);
            const float dx = __int_as_float(rec[0]);
            const int qs = rec[1];
#pragma unroll
            for (int rp = 0; rp < RP; ++rp) {
              const int64_t blk = (int64_t)min(row0 + 4 * rp, H - 1) * nbi + j;
              const u32x4 wb = load_stream16(dq + blk * 16);
              const float db = f16_bits_to_f32(load_stream2(dd + blk));
              v[rp] += down_block_value(wb, db, xa, xb, dx, qs);
            }
          }
          store_dots(pp[c], v);
        }
      }
    }
  };
  pair_group(0);
  for (int r0 = NP; r0 < np; r0 += NP) pair_group(r0);  // uniform
  MMV_TL_END(kTlDownPart, 2);
}

// Y[b][n] = tree_j (w[b k + j] dot_{b k + j}[n]) + s_b dot_{Bk + b}[n] with
// the sum K3 forms (down_combine_tree); pairs with ids outside [0, E) add
// zero.  grid = (ceil(H / 256), B).
template <int B>  // B = 0: rows at run time
__global__ __launch_bounds__(256) void k_moe_combine(MoeArgs a) {
  const mmv_moe_layer &L = a.L;
  const int H = L.hidden, k = L.top_k, E = L.n_experts, Bk = (B > 0 ? B : a.nrows) * k;
  const int b = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
  const int nc = min(n, H - 1);
  MMV_TL(0);
  const bool has_sh = L.sh_down_qs != nullptr;
  static_assert(MMV_MAX_TOPK <= 16, "slots per row");
  float d[16], pr[16];
  // every load first, unconditionally (pinned in registers, so that the
  // selects below cannot pull them into branches one round trip each)
#pragma unroll
  for (int j = 0; j < 16; ++j) d[j] = a.dpart[(int64_t)(b * k + min(j, k - 1)) * H + nc];
  float dsh = a.dpart[(int64_t)(has_sh ? Bk + b : 0) * H + nc];
#pragma unroll
  for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(d[j]));
  asm volatile("" : "+v"(dsh));
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int p = b * k + min(j, k - 1);
    const int e = a.ids[p];
    pr[j] = j < k ? a.weights[p] * ((e >= 0 && e < E) ? d[j] : 0.0f) : 0.0f;
  }
  float v = down_combine_tree(pr);
  if (has_sh) v = fmaf(a.shared_w ? a.shared_w[b] : 1.0f, dsh, v);
  if (n < H) a.Y[(int64_t)b * a.ldy + n] = v;
  if (b == 0) MMV_TL_END(kTlCombine, 1);
  if (a.has_dbg && a.dbg.down_out && n < H) {  // each pair's product, unweighted
    for (int j = 0; j < k; ++j) {
      const int e = a.ids[b * k + j];
      a.dbg.down_out[(int64_t)(b * k + j) * H + n] = (e >= 0 && e < E) ? d[j] : 0.0f;
    }
    if (has_sh) a.dbg.down_out[(int64_t)(Bk + b) * H + n] = dsh;
  }
}

// ---------------------------------------------------------------------------
// Verify / prefill batches: 8 < B <= 64 rows
// ---------------------------------------------------------------------------
// "Flash-Next on Strix Halo" (Expert GEMMs) builds per-expert row lists in a
// prepass and dispatches compact (expert, tile) work, so that each expert's
// weights are read once for all the rows that chose it.  Here: the router
// (every row in one launch for H of 1024 or 2048, else 8 rows per launch),
// top-k a wave per row, the row lists and one work record per (expert,
// 8-row group) by one workgroup (k_moe_gather_rows), gate/up by (record,
// 32-row tile) workgroups (the same tile code as B <= 8, an expert's
// weights re-read from cache for each further 8 rows), then the by-expert
// down projection and the combine with the row count at run time.  Every
// row is formed by the same arithmetic as for B <= 8, so it is the same bits.

// top-k for every row (layer decode): a workgroup per 4 rows, a wave per row
__global__ __launch_bounds__(256) void k_moe_topk_rows(MoeArgs a) {
  const mmv_moe_layer &L = a.L;
  const int E = L.n_experts, k = L.top_k, b0 = blockIdx.x * 4;
  topk_any(a.logits + (int64_t)b0 * (E + 1), E + 1, E, min(4, a.nrows - b0), k,
           L.shared_gate_row ? 1 : 0, a.ids_out + (int64_t)b0 * k,
           a.weights_out + (int64_t)b0 * k, a.shared_w_out + b0);
}

// Row lists for B <= 64 (B * k <= 1024 pairs, E <= 1024) by counting over
// the experts: each expert's 64-bit mask of the rows that chose it (LDS
// atomics), then prefix sums over the experts (a thread per expert) give
// its first list position and its group number, and pair (b, j) of expert
// e goes to start[e] + (rows below b in mask[e]): grouped by expert, then
// by row, as the rank sort of build_gather orders them (a valid row meets
// an expert once).  Ids outside [0, E) take no part; a row naming one
// expert twice (invalid) keeps one of the two pairs.  One workgroup of
// 1024 threads.
__global__ __launch_bounds__(1024) void k_moe_gather_rows(MoeArgs a) {
  __shared__ unsigned long long s_mask[MMV_MAX_EXPERTS];
  __shared__ int s_start[MMV_MAX_EXPERTS];
  __shared__ int s_item[MMV_MAX_EXPERTS];  // the expert's first work record
  __shared__ int s_wc[16], s_wp[16], s_wg[16];
  const mmv_moe_layer &L = a.L;
  const int t = threadIdx.x, E = L.n_experts, k = L.top_k, Bk = a.nrows * k;
  const int lane = t & 63, wv = t >> 6;
  if (t < E) s_mask[t] = 0ull;
  __syncthreads();
  if (t < Bk) {
    const int e = a.ids[t];
    if (e >= 0 && e < E) atomicOr(&s_mask[e], 1ull << (t / k));
  }
  __syncthreads();
  const unsigned long long m = t < E ? s_mask[t] : 0ull;
  const int c = __popcll(m), pr = c > 0 ? 1 : 0;
  const int g = (c + MMV_MAX_BATCH - 1) / MMV_MAX_BATCH;  // gate/up row groups
  int ic = c, ip = pr, ig = g;  // inclusive prefix sums within the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int oc = __shfl_up(ic, d), op = __shfl_up(ip, d), og = __shfl_up(ig, d);
    if (lane >= d) { ic += oc; ip += op; ig += og; }
  }
  if (lane == 63) { s_wc[wv] = ic; s_wp[wv] = ip; s_wg[wv] = ig; }
  __syncthreads();
  int bc = 0, bp = 0, bg = 0, tc = 0, tp = 0, tg = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int wc = s_wc[w], wp = s_wp[w], wg = s_wg[w];
    bc += w < wv ? wc : 0;
    bp += w < wv ? wp : 0;
    bg += w < wv ? wg : 0;
    tc += wc;
    tp += wp;
    tg += wg;
  }
  const int start = bc + ic - c, urank = bp + ip - pr, gstart = bg + ig - g;  // exclusive
  // work records: the shared expert's row groups, then each routed expert's
  // (record = expert, or -1 for the shared one; rows; up to 8 pair indices
  // as int16 pairs).  Gate/up reads one record, with nothing before it.
  const int nsh = a.routed_shared ? (a.nrows + MMV_MAX_BATCH - 1) / MMV_MAX_BATCH : 0;
  int32_t *rec0 = a.work + kWorkRecInts;
  if (t < nsh) {
    int32_t *rec = rec0 + kWorkRecInts * t;
    const int r0 = MMV_MAX_BATCH * t, nr = min(MMV_MAX_BATCH, a.nrows - r0);
    rec[0] = -1;
    rec[1] = nr;
#pragma unroll
    for (int i = 0; i < MMV_MAX_BATCH / 2; ++i) {  // pair of row r: Bk + r
      const int pa = Bk + r0 + min(2 * i, nr - 1), pb = Bk + r0 + min(2 * i + 1, nr - 1);
      rec[2 + i] = (pa & 0xFFFF) | (pb << 16);
    }
  }
  if (t < E) {
    s_item[t] = nsh + gstart;
    if (pr)
      for (int q = 0; q < g; ++q) {
        int32_t *rec = rec0 + kWorkRecInts * (nsh + gstart + q);
        rec[0] = t;
        rec[1] = min(MMV_MAX_BATCH, c - MMV_MAX_BATCH * q);
      }
  }
  if (t == 0) a.work[0] = nsh + tg;
  int32_t *gl = a.gather;
  const bool dbg = a.has_dbg != 0;
  if (t < E) {
    s_start[t] = start;
    if (pr) {
      gl[1 + urank] = t;
      gl[1 + Bk + urank] = start;
      if (dbg && a.dbg.unique) a.dbg.unique[urank] = t;
      if (dbg && a.dbg.offsets) a.dbg.offsets[urank] = start;
    }
  }
  if (t == 0) {
    gl[0] = tp;
    gl[1 + Bk + tp] = tc;
    if (dbg && a.dbg.offsets) a.dbg.offsets[tp] = tc;
    if (dbg && a.dbg.n_unique) a.dbg.n_unique[0] = tp;
  }
  __syncthreads();
  if (t < Bk) {
    const int e = a.ids[t];
    if (e >= 0 && e < E) {
      const int rank = __popcll(s_mask[e] & ((1ull << (t / k)) - 1ull)), pos = s_start[e] + rank;
      gl[2 + 2 * Bk + pos] = t;
      int16_t *rp = reinterpret_cast<int16_t *>(rec0 + kWorkRecInts * (s_item[e] + rank / MMV_MAX_BATCH) + 2);
      rp[rank % MMV_MAX_BATCH] = (int16_t)t;
      if (dbg && a.dbg.pairs) a.dbg.pairs[pos] = t;
    }
  }
}

// gate/up for B <= 64: one workgroup per (work item, 32-row tile), a work
// item being up to eight rows of one expert (k_moe_gather_rows writes one
// record per item, the shared expert's row groups first, then each routed
// expert's: the expert, the row count and the rows' pair indices, so that
// the weights go out after one round trip); items past the published count
// exit.  The B <= 8 tile code does the rows; SC:
// every scale plane 16-byte aligned (checked on the host), the scales fetched
// as 16-byte chunks.
template <int T, bool SC>
__global__ __launch_bounds__(256) void k_moe_gate_up_rows(MoeArgs a) {
  __shared__ int rowmap[MMV_MAX_BATCH];
  __shared__ int pairmap[MMV_MAX_BATCH];
  __shared__ float hbuf[MMV_MAX_BATCH][32];
  extern __shared__ __align__(16) uint8_t smem[];
  const mmv_moe_layer &L = a.L;
  const int k = L.top_k, I = L.inter, B = a.nrows, Bk = B * k;
  const int ntiles = I >> 5;
  const int wi = blockIdx.x / ntiles, tile = blockIdx.x - wi * ntiles;
  // the count and this item's record in one round trip (wi is below the
  // record capacity, so the record is in bounds even past the count)
  const int32_t *rec = a.work + kWorkRecInts * (1 + wi);
  const int W = a.work[0];
  const int e = rec[0], nc = rec[1];
  int32_t pw[MMV_MAX_BATCH / 2];
#pragma unroll
  for (int i = 0; i < MMV_MAX_BATCH / 2; ++i) pw[i] = rec[2 + i];
  if (wi >= W || nc <= 0 || nc > MMV_MAX_BATCH) return;  // uniform; never for a published item
  const bool shared_slot = e < 0;
  const uint8_t *gq, *uq;
  const uint16_t *gd, *ud;
  if (shared_slot) {
    gq = L.sh_gate_qs; gd = L.sh_gate_d; uq = L.sh_up_qs; ud = L.sh_up_d;
  } else {
    expert_gate_up(L, e, gq, gd, uq, ud);
  }
  int ncv = nc;  // opaque: with its range known the compiler unrolls per row count
  asm volatile("" : "+s"(ncv));
  if (threadIdx.x < (unsigned)nc) {
    const int tr = threadIdx.x;
    int32_t two = pw[0];
#pragma unroll
    for (int i = 1; i < MMV_MAX_BATCH / 2; ++i) two = (tr >> 1) == i ? pw[i] : two;
    const int p = (tr & 1) ? (two >> 16) : (int)(int16_t)(two & 0xFFFF);
    pairmap[tr] = p;
    rowmap[tr] = shared_slot ? p - Bk : p / k;
  }
  const XPre<1> none{};
  gate_up_tile<MMV_MAX_BATCH, T, 0, SC, 4>(a, gq, gd, uq, ud, tile, ncv, rowmap, pairmap, smem,
                                        hbuf, none, []() {});
}

namespace {

MoeArgs make_args(const mmv_moe_layer &L, const float *X, int64_t ldx, int B,
                  const int32_t *ids, const float *weights, const float *shared_w, float *Y,
                  int64_t ldy, uint8_t *ws, const mmv_moe_debug *dbg) {
  MoeArgs a;
  a.L = L;
  // expert strides resolved here: the kernels always step by them
  const int64_t nb = (int64_t)L.inter * (L.hidden / 32);
  auto fix = [](int64_t &st, int64_t dflt) { if (st == 0) st = dflt; };
  fix(a.L.gate_qs_stride, 16 * nb);
  fix(a.L.up_qs_stride, 16 * nb);
  fix(a.L.down_qs_stride, 16 * nb);
  fix(a.L.gate_d_stride, nb);
  fix(a.L.up_d_stride, nb);
  fix(a.L.down_d_stride, nb);
  a.X = X;
  a.ldx = ldx;
  a.ids = ids;
  a.weights = weights;
  a.shared_w = shared_w;
  a.Y = Y;
  a.ldy = ldy;
  const bool has_sh = L.sh_gate_qs != nullptr;
  const MoeWsLayout lay = moe_ws_layout(L.n_experts, L.hidden, L.inter, L.top_k, B, has_sh);
  a.hq = ws + lay.hq;
  a.gather = reinterpret_cast<int32_t *>(ws + lay.gather);
  a.P = B * L.top_k + (has_sh ? B : 0);
  a.routed_shared = has_sh ? 1 : 0;
  a.has_dbg = dbg != nullptr;
  a.dbg = dbg ? *dbg : mmv_moe_debug{};
  a.logits = reinterpret_cast<float *>(ws + lay.logits);
  a.dpart = reinterpret_cast<float *>(ws + lay.dpart);
  a.nrows = B;
  a.work = reinterpret_cast<int32_t *>(ws + lay.work);
  a.gather_ready = 0;
  a.ids_out = nullptr;
  a.weights_out = nullptr;
  a.shared_w_out = nullptr;
  a.router_wgs = 0;
  a.topk_in_k2 = 0;
  return a;
}

template <int B, int T>
void launch_gate_up(const MoeArgs &a, hipStream_t s) {
  const int slots = B * a.L.top_k + (a.routed_shared ? 1 : 0);
  const int ntiles = a.L.inter / 32;
  const size_t lds = xstage_bytes(B, a.L.hidden);
  // 8 waves of 4 rows per matrix for 3..6 rows: half the weight registers
  // (93 VGPRs against 129-149), five waves per SIMD instead of three; E = 512
  // us per layer, B = 3 / 4 / 5 / 6: 32.2 / 36.7 / 40.7 / 43.8 ->
  // 31.0 / 35.2 / 40.5 / 42.7; level at B = 7 and 8
  constexpr int NW = (B >= 3 && B <= 6 && T > 0) ? 8 : 4;
  hipLaunchKernelGGL((k_moe_gate_up<B, T, NW>), dim3(slots * ntiles), dim3(64 * NW), lds, s, a);
}

// waves per workgroup: the 4 output rows' experts are split over them by id;
// 8 waves measured faster at B = 4 (E = 512: 38.9 against 39.6 us per
// layer), slower at B = 8 (registers then allow one workgroup per CU) and at
// B <= 2 (E = 256, B = 1: 19.3 against 15.7 us; E = 512, B = 2: 29.9 against
// 24.9 us)
template <int B>
constexpr int down_waves() { return (B == 3 || B == 4) ? 8 : 4; }

// rows from which the down projection runs by expert (two launches: the
// per-pair products, then the combine)
constexpr int kDownSplitMinB = 3;

template <int B, int TI>
void launch_down(const MoeArgs &a, hipStream_t s) {
  const int knob = path_switch(MMV_PATH_MOE_DOWN);
  // the one-kernel path stages Q8_1(h) of all P pairs in LDS: only where it fits
  const bool fits = (int64_t)a.P * a.L.inter <= kMaxDownStageElems;
  if (!fits || knob == 2 || (knob != 1 && B >= kDownSplitMinB)) {
    const int slots = min(a.L.n_experts, B * a.L.top_k) + (a.L.sh_down_qs ? 1 : 0);
    const int ntile = (a.L.hidden + kDownPartRows - 1) / kDownPartRows;
    hipLaunchKernelGGL((k_moe_down_part<B, TI>), dim3(slots * ntile), dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_moe_combine<B>), dim3((a.L.hidden + 255) / 256, B), dim3(256), 0, s, a);
    return;
  }
  const size_t lds = xstage_bytes(a.P, a.L.inter);
  constexpr int NWV = down_waves<B>();
  hipLaunchKernelGGL((k_moe_down<B, TI, NWV>), dim3((a.L.hidden + 3) / 4), dim3(64 * NWV), lds, s,
                     a);
}

// one router row (one wave) per workgroup: the E + 1 rows spread over every
// CU (E = 256, B = 1: the gate/up kernel starts 0.4 us earlier than with
// four rows per workgroup; at E = 512 the rows outnumber the CUs anyway)
template <int B, int HC>
void launch_router_k1(const MoeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((k_moe_router<B, HC>), dim3(a.router_wgs), dim3(64), 0, s, a);
}

template <int B>
void launch_experts(const MoeArgs &a, hipStream_t s) {
  switch (a.L.hidden) {
    case 512: launch_gate_up<B, 1>(a, s); break;
    case 1024: launch_gate_up<B, 2>(a, s); break;
    case 2048: launch_gate_up<B, 4>(a, s); break;
    case 4096: launch_gate_up<B, 8>(a, s); break;
    default: launch_gate_up<B, 0>(a, s); break;
  }
  switch (a.L.inter) {
    case 512: launch_down<B, 1>(a, s); break;
    case 1024: launch_down<B, 2>(a, s); break;
    default: launch_down<B, 0>(a, s); break;
  }
}

// work items: (shared row groups) + U + sum over experts of (ceil(c_e / 8) - 1)
// <= (shared row groups) + U + (B*k - U) / 8 (c_e rows chose expert e, the
// c_e sum to B*k), which does not fall as U grows: bounded at U = min(E, B*k)
int rows_work_max(const MoeArgs &a) {
  const int Bk = a.nrows * a.L.top_k, Umax = min(a.L.n_experts, Bk);
  return (a.routed_shared ? (a.nrows + MMV_MAX_BATCH - 1) / MMV_MAX_BATCH : 0) + Umax +
         (Bk - Umax) / MMV_MAX_BATCH;
}

// every gate / up scale plane 16-byte aligned: the experts' planes start
// at multiples of their d stride (2 bytes per element) from the layer's
bool rows_scales16(const MoeArgs &a) {
  const mmv_moe_layer &L = a.L;
  auto al = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool sh = !a.routed_shared || (al(L.sh_gate_d) && al(L.sh_up_d));
  return al(L.gate_d) && al(L.up_d) && sh && (L.gate_d_stride * 2) % 16 == 0 &&
         (L.up_d_stride * 2) % 16 == 0;
}

template <int T>
void launch_gate_up_rows(const MoeArgs &a, hipStream_t s) {
  const dim3 grid(rows_work_max(a) * (a.L.inter / 32)), block(256);
  const size_t lds = xstage_bytes(MMV_MAX_BATCH, a.L.hidden);
  if (T > 0 && rows_scales16(a))
    hipLaunchKernelGGL((k_moe_gate_up_rows<T, T != 0>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((k_moe_gate_up_rows<T, false>), grid, block, lds, s, a);
}

template <int TI>
void launch_down_rows(const MoeArgs &a, hipStream_t s) {
  const int slots = min(a.L.n_experts, a.nrows * a.L.top_k) + (a.L.sh_down_qs ? 1 : 0);
  const int ntile = (a.L.hidden + kDownPartRows - 1) / kDownPartRows;
  hipLaunchKernelGGL((k_moe_down_part<0, TI>), dim3(slots * ntile), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_moe_combine<0>), dim3((a.L.hidden + 255) / 256, a.nrows), dim3(256), 0,
                     s, a);
}

// B > 8: the row lists (unless published), gate/up, down by expert, combine
void launch_experts_rows(const MoeArgs &a, hipStream_t s) {
  if (!a.gather_ready) hipLaunchKernelGGL(k_moe_gather_rows, dim3(1), dim3(1024), 0, s, a);
  switch (a.L.hidden) {
    case 512: launch_gate_up_rows<1>(a, s); break;
    case 1024: launch_gate_up_rows<2>(a, s); break;
    case 2048: launch_gate_up_rows<4>(a, s); break;
    case 4096: launch_gate_up_rows<8>(a, s); break;
    default: launch_gate_up_rows<0>(a, s); break;
  }
  switch (a.L.inter) {
    case 512: launch_down_rows<1>(a, s); break;
    case 1024: launch_down_rows<2>(a, s); break;
    default: launch_down_rows<0>(a, s); break;
  }
}

template <int B>
void launch_route(const MoeArgs &a, hipStream_t s) {
  switch (a.L.hidden) {
    case 1024: launch_router_k1<B, 4>(a, s); break;
    case 2048: launch_router_k1<B, 8>(a, s); break;
    case 4096: launch_router_k1<B, 16>(a, s); break;
    default: launch_router_k1<B, 0>(a, s); break;
  }
}

}  // namespace

hipError_t run_moe_experts(const mmv_moe_layer &L, const float *X, int64_t ldx, int B,
                           const int32_t *ids, const float *weights, const float *shared_w,
                           float *Y, int64_t ldy, uint8_t *ws, const mmv_moe_debug *dbg,
                           hipStream_t s) {
  const MoeArgs a = make_args(L, X, ldx, B, ids, weights, shared_w, Y, ldy, ws, dbg);
  if (dbg && dbg->x_q8) {  // Q8_1(x) by the routine the gate/up workgroups stage x with
    const hipError_t e = run_quantize_q8_1(X, L.hidden, ldx, B,
                                           static_cast<uint8_t *>(dbg->x_q8), s);
    if (e != hipSuccess) return e;
  }
  if (B > MMV_MAX_BATCH) {
    launch_experts_rows(a, s);
    return hipGetLastError();
  }
  switch (B) {
    case 1: launch_experts<1>(a, s); break;
    case 2: launch_experts<2>(a, s); break;
    case 3: launch_experts<3>(a, s); break;
    case 4: launch_experts<4>(a, s); break;
    case 5: launch_experts<5>(a, s); break;
    case 6: launch_experts<6>(a, s); break;
    case 7: launch_experts<7>(a, s); break;
    case 8: launch_experts<8>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t run_moe_layer(const mmv_moe_layer &L, const float *X, int64_t ldx, int B,
                         int32_t *ids, float *weights, float *Y, int64_t ldy, uint8_t *ws,
                         hipStream_t s) {
  const bool has_sh = L.sh_gate_qs != nullptr;
  const MoeWsLayout lay = moe_ws_layout(L.n_experts, L.hidden, L.inter, L.top_k, B, has_sh);
  float *sw = reinterpret_cast<float *>(ws + lay.shared_w);
  MoeArgs a = make_args(L, X, ldx, B, ids, weights, sw, Y, ldy, ws, nullptr);
  a.ids_out = ids;
  a.weights_out = weights;
  a.shared_w_out = sw;
  a.router_wgs = L.n_experts + (L.shared_gate_row ? 1 : 0);
  // Top-k in every gate/up workgroup costs no launch and is cheapest for
  // one or two rows; for more rows it grows with B in every workgroup, and
  // one workgroup of its own (plus a launch) costs less.  A grid-wide
  // barrier or ticket inside one kernel measured slower than a launch.
  if (B > MMV_MAX_BATCH) {
    // router rows 8 activation rows at a time, top-k a wave per row, then
    // the row lists and the experts
    const int E = L.n_experts;
    const bool one = launch_router_lds(L.router, E, L.hidden, L.shared_gate_row, X, ldx, B,
                                       a.logits, s);
    for (int b0 = one ? B : 0; b0 < B; b0 += MMV_MAX_BATCH) {
      MoeArgs ac = a;
      ac.X = X + (int64_t)b0 * ldx;
      ac.logits = a.logits + (int64_t)b0 * (E + 1);
      switch (min(B - b0, MMV_MAX_BATCH)) {
        case 1: launch_route<1>(ac, s); break;
        case 2: launch_route<2>(ac, s); break;
        case 3: launch_route<3>(ac, s); break;
        case 4: launch_route<4>(ac, s); break;
        case 5: launch_route<5>(ac, s); break;
        case 6: launch_route<6>(ac, s); break;
        case 7: launch_route<7>(ac, s); break;
        default: launch_route<8>(ac, s); break;
      }
    }
    hipLaunchKernelGGL(k_moe_topk_rows, dim3((B + 3) / 4), dim3(256), 0, s, a);
    launch_experts_rows(a, s);
    return hipGetLastError();
  }
  const int knob = path_switch(MMV_PATH_MOE_TOPK);
  a.topk_in_k2 = knob > 0 ? 0 : (knob < 0 ? 1 : (B <= 2 ? 1 : 0));
  a.gather_ready = a.topk_in_k2 ? 0 : 1;
  switch (B) {
#define MMV_LAYER_CASE(BB)                                                              \
  case BB:                                                                              \
    if (!launch_router_lds(L.router, L.n_experts, L.hidden, L.shared_gate_row, X, ldx, BB, \
                           a.logits, s))                                                \
      launch_route<BB>(a, s);                                                           \
    if (!a.topk_in_k2) hipLaunchKernelGGL((k_moe_topk_gather<BB>), dim3(1), dim3(64 * BB), 0, s, a); \
    launch_experts<BB>(a, s);                                                           \
    break;
    MMV_LAYER_CASE(1) MMV_LAYER_CASE(2) MMV_LAYER_CASE(3) MMV_LAYER_CASE(4)
    MMV_LAYER_CASE(5) MMV_LAYER_CASE(6) MMV_LAYER_CASE(7) MMV_LAYER_CASE(8)
#undef MMV_LAYER_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mmv

// Timeline of the last MoE launches (timeline builds only): copies the stamp
// array ([7 kinds][4096 workgroups][8 points] uint64 of the 100 MHz clock,
// 0 where nothing was noted) to dst if dst is given, then clears it if
// `clear`.  Returns the array's size in bytes, or 0 in the normal build.
extern "C" size_t mmv_timeline(void *dst, int clear, void *stream) {
#ifdef MMV_TIMELINE
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void *addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(mmv::g_timeline)) != hipSuccess) return 0;
  if (dst && hipMemcpyAsync(dst, addr, sizeof(mmv::g_timeline), hipMemcpyDeviceToDevice, s) !=
                 hipSuccess)
    return 0;
  if (clear && hipMemsetAsync(addr, 0, sizeof(mmv::g_timeline), s) != hipSuccess) return 0;
  return sizeof(mmv::g_timeline);
#else
  (void)dst;
  (void)clear;
  (void)stream;
  return 0;
#endif
}
