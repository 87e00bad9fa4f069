// moe.hip -- the mixture-of-experts decode path: F32 router, softmax +
// top-k, per-expert row lists, gate/up with SiLU and a Q8_1 epilogue, and
// the down projection with the weighted combine and the shared expert.
//
// "Fourteen hours to 100 tokens per second" traces one decode token as
// separate kernel classes (F32 router, top-k routing, mul_mat_id expert
// matvecs, quantize_q8_1, broadcast glue) and removes glue by fusion: the
// top-k kernel writes ids and weights directly, silu(gate)*up is quantized
// to Q8 in the producing kernel, and the K <= 512 down projection uses four
// rows per wave.  "Flash-Next on Strix Halo" (Expert GEMMs) builds
// per-expert row lists so each expert's weights are read once for all rows
// that chose it.  Here, on gfx950:
//  - router: one wave per router row, 128-bit fp32 loads, fp32 sums;
//  - top-k: one wave per token row; order-preserving 64-bit keys
//    (value, ~index) make equal logits rank by lower index; the weights are
//    exp(l - l_max) over the selected k, renormalised (the softmax
//    denominator over all E cancels);
//  - every expert workgroup rebuilds the row lists of the B*k (row, slot)
//    pairs in LDS from ids (<= 128 entries), so routing stays on the device
//    and the launch sequence can be captured in a HIP graph;
//  - gate/up: a workgroup owns 32 consecutive rows of one expert's gate and
//    up, so silu(g)*u of those rows forms exactly one Q8_1 block of the
//    down projection's input, quantized in the epilogue;
//  - down: each output row is owned by one 16-lane group that walks the
//    unique experts in ascending id, then the shared expert, accumulating
//    per-row partials in a fixed order; no atomics, one store per output.
#include "common.hpp"
#include "launch.hpp"
#include "q4_0.hpp"
#include "q8_1.hpp"
#include "layout.hpp"

namespace mmv {

constexpr int kMaxPairs = MMV_MAX_BATCH * MMV_MAX_TOPK;  // 128

// ---------------------------------------------------------------------------
// router logits: logits[b*(E+1) + e], e in [0, E] (row E = shared gate row)
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(64) void k_router(const float *__restrict__ R, int E, int H,
                                               const float *__restrict__ shg,
                                               const float *__restrict__ X, int64_t ldx,
                                               float *__restrict__ logits) {
  const int e = blockIdx.x;
  const float *row = e < E ? R + (int64_t)e * H : shg;
  const int lane = threadIdx.x;
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  const int nc = H >> 2;
#pragma unroll 4
  for (int c = lane; c < nc; c += 64) {
    const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row) + c);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const f32x4 x = load_f4(X + (int64_t)b * ldx + 4 * c);
      acc[b] = fmaf(r.x, x.x, acc[b]);
      acc[b] = fmaf(r.y, x.y, acc[b]);
      acc[b] = fmaf(r.z, x.z, acc[b]);
      acc[b] = fmaf(r.w, x.w, acc[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float v = group_sum<64>(acc[b]);
    if (lane == 0) logits[(int64_t)b * (E + 1) + e] = v;
  }
}

// ---------------------------------------------------------------------------
// top-k + renormalised weights: one wave per token row
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  v = v + 0.0f;  // -0 and +0 compare equal: map both to +0
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t oh = __shfl_xor(hi, m, kWave), ol = __shfl_xor(lo, m, kWave);
    if (oh > hi || (oh == hi && ol > lo)) { hi = oh; lo = ol; }
  }
  return ((uint64_t)hi << 32) | lo;
}

constexpr int kKeysPerLane = MMV_MAX_EXPERTS / 64;  // 16

__global__ __launch_bounds__(512) void k_topk(const float *__restrict__ L, int64_t ldl, int E,
                                              int B, int k, int has_shared,
                                              int32_t *__restrict__ ids,
                                              float *__restrict__ weights,
                                              float *__restrict__ shared_w) {
  const int b = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (b >= B) return;
  const float *l = L + (int64_t)b * ldl;
  uint64_t key[kKeysPerLane];
#pragma unroll
  for (int i = 0; i < kKeysPerLane; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? topk_key(l[e], e) : 0ull;  // 0 never wins: real keys are > 0
  }
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(~(uint32_t)best);
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
    if (lane == j) my_id = e;
  }
  const float lmax = l[__shfl(my_id, 0, kWave)];
  const float ex = lane < k ? expf(l[my_id] - lmax) : 0.0f;
  const float den = group_sum<16>(ex);  // k <= 16: lanes 0..15
  if (lane < k) {
    ids[(int64_t)b * k + lane] = my_id;
    weights[(int64_t)b * k + lane] = ex / den;
  }
  if (lane == 0 && shared_w)
    shared_w[b] = has_shared ? 1.0f / (1.0f + expf(-l[E])) : 1.0f;
}

hipError_t run_moe_route(const float *router, int E, int H, const float *X, int64_t ldx,
                         int B, int k, const float *shg, float *logits, int32_t *ids,
                         float *weights, float *shared_w, hipStream_t s) {
  const float *L = X;
  int64_t ldl = ldx;
  if (router) {
    const int rows = E + (shg ? 1 : 0);
    switch (B) {
#define MMV_ROUTER_CASE(BB) \
  case BB: hipLaunchKernelGGL(k_router<BB>, dim3(rows), dim3(64), 0, s, router, E, H, shg, X, ldx, logits); break;
      MMV_ROUTER_CASE(1) MMV_ROUTER_CASE(2) MMV_ROUTER_CASE(3) MMV_ROUTER_CASE(4)
      MMV_ROUTER_CASE(5) MMV_ROUTER_CASE(6) MMV_ROUTER_CASE(7) MMV_ROUTER_CASE(8)
#undef MMV_ROUTER_CASE
      default: return hipErrorInvalidValue;
    }
    L = logits;
    ldl = E + 1;
  }
  hipLaunchKernelGGL(k_topk, dim3(1), dim3(64 * B), 0, s, L, ldl, E, B, k,
                     (router && shg) ? 1 : 0, ids, weights, shared_w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// per-expert row lists, rebuilt in LDS by every expert workgroup
// ---------------------------------------------------------------------------
struct GatherLds {
  int sid[kMaxPairs];      // ids, or -1 for an id outside [0, E)
  int first[kMaxPairs];    // 1 if the first occurrence of its expert
  int unique[kMaxPairs];   // sorted unique experts
  int offsets[kMaxPairs + 1];
  int pairs[kMaxPairs];    // b*k + j grouped by expert, then b, then j
  int U;
};

// blockDim.x >= Bk; contains __syncthreads (call from uniform control flow)
__device__ void build_gather(const int32_t *__restrict__ ids, int Bk, int E, GatherLds &g) {
  const int t = threadIdx.x;
  if (t < Bk) {
    const int e = ids[t];
    g.sid[t] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  if (t < Bk) {
    const int e = g.sid[t];
    int first = e >= 0;
    for (int t2 = 0; t2 < t; ++t2) first &= (g.sid[t2] != e);
    g.first[t] = first;
  }
  __syncthreads();
  if (t < Bk) {
    const int e = g.sid[t];
    if (e >= 0) {
      int urank = 0, nless = 0, before = 0;
      for (int t2 = 0; t2 < Bk; ++t2) {
        const int v = g.sid[t2];
        if (v >= 0 && v < e) { ++nless; urank += g.first[t2]; }
        before += (v == e && t2 < t);
      }
      g.pairs[nless + before] = t;
      if (g.first[t]) { g.unique[urank] = e; g.offsets[urank] = nless; }
    }
  }
  if (t == 0) {
    int U = 0, nv = 0;
    for (int t2 = 0; t2 < Bk; ++t2) { U += g.first[t2]; nv += g.sid[t2] >= 0; }
    g.U = U;
    g.offsets[U] = nv;
  }
  __syncthreads();
}

// Workspace view: Q8_1 of h for P pairs (planar), then integer code sums.
struct HqView {
  uint8_t *codes;    // [P][I]
  uint16_t *ds;      // [P][I/32][2]
  int *qsum;         // [P][I/32]
};
__device__ inline HqView hq_view(uint8_t *base, int P, int I) {
  HqView v;
  v.codes = base;
  v.ds = reinterpret_cast<uint16_t *>(base + (size_t)P * I);
  v.qsum = reinterpret_cast<int *>(base + (size_t)P * I + (size_t)4 * P * (I / 32));
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
  int P;             // pairs: B*k (+ B with a shared expert)
  mmv_moe_debug dbg;
  int has_dbg;
};

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// gate/up + SiLU + Q8_1 epilogue.  grid = (B*k + shared) slots x (I/32) tiles.
// 4 waves; wave w owns rows 8w..8w+7 of the tile in both gate and up;
// 16 lanes per row (4 rows per pass), passes: gate lo/hi, up lo/hi.
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(256) void k_moe_gate_up(MoeArgs a) {
  __shared__ GatherLds g;
  __shared__ int rowmap[MMV_MAX_BATCH];
  __shared__ int pairmap[MMV_MAX_BATCH];
  __shared__ float hbuf[MMV_MAX_BATCH][32];
  extern __shared__ __align__(16) uint8_t smem[];

  const mmv_moe_layer &L = a.L;
  const int k = L.top_k, H = L.hidden, I = L.inter;
  const int Bk = B * k;
  const int ntiles = I >> 5;
  const int slot = blockIdx.x / ntiles, tile = blockIdx.x - slot * ntiles;
  const bool has_sh = L.sh_gate_qs != nullptr;

  build_gather(a.ids, Bk, L.n_experts, g);
  if (blockIdx.x == 0 && a.has_dbg) {
    const int t = threadIdx.x;
    if (a.dbg.unique && t < g.U) a.dbg.unique[t] = g.unique[t];
    if (a.dbg.offsets && t <= g.U) a.dbg.offsets[t] = g.offsets[t];
    if (a.dbg.pairs && t < g.offsets[g.U]) a.dbg.pairs[t] = g.pairs[t];
    if (a.dbg.n_unique && t == 0) a.dbg.n_unique[0] = g.U;
  }
  const bool shared_slot = has_sh && slot == Bk;
  if (!shared_slot && slot >= g.U) return;  // uniform over the workgroup

  const int nbh = H >> 5;
  const uint8_t *gq, *uq;
  const uint16_t *gd, *ud;
  int nr;
  if (shared_slot) {
    gq = L.sh_gate_qs; gd = L.sh_gate_d; uq = L.sh_up_qs; ud = L.sh_up_d;
    nr = B;
  } else {
    const int64_t e = g.unique[slot];
    const int64_t eo = e * I * nbh;
    gq = L.gate_qs + eo * 16; gd = L.gate_d + eo;
    uq = L.up_qs + eo * 16; ud = L.up_d + eo;
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

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int sub = lane & 15, q = lane >> 4;
  // pass p: 0,1 gate rows (4p + q), 2,3 up rows (4(p-2) + q) of this wave's 8
  int64_t rowoff[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int n = tile * 32 + 8 * wv + 4 * (p & 1) + q;
    rowoff[p] = (int64_t)n * nbh;
  }
  // first weight blocks in flight before staging x
  u32x4 w0[4];
  float d0[4];
  const int j0 = sub < nbh ? sub : 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint8_t *wq = p < 2 ? gq : uq;
    const uint16_t *wd = p < 2 ? gd : ud;
    w0[p] = load_stream16(wq + (rowoff[p] + j0) * 16);
    d0[p] = f16_bits_to_f32(load_stream2(wd + rowoff[p] + j0));
  }
  __syncthreads();  // rowmap / pairmap visible
  const XStage st = xstage_at(smem, B, H);
  stage_quantize(a.X, a.ldx, rowmap, nr, H, st);
  __syncthreads();

  float acc[4][B];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int r = 0; r < B; ++r) acc[p][r] = 0.0f;

  for (int j = sub; j < nbh; j += 16) {
    u32x4 w[4];
    float dw[4];
    if (j == sub) {
#pragma unroll
      for (int p = 0; p < 4; ++p) { w[p] = w0[p]; dw[p] = d0[p]; }
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint8_t *wq = p < 2 ? gq : uq;
        const uint16_t *wd = p < 2 ? gd : ud;
        w[p] = load_stream16(wq + (rowoff[p] + j) * 16);
        dw[p] = f16_bits_to_f32(load_stream2(wd + rowoff[p] + j));
      }
    }
#pragma unroll
    for (int r = 0; r < B; ++r) {
      if (r < nr) {
        const int8_t *xc = st.codes + (size_t)r * H + 32 * j;
        const i32x4 xa = *reinterpret_cast<const i32x4 *>(xc);
        const i32x4 xb = *reinterpret_cast<const i32x4 *>(xc + 16);
        const int xs = st.qsum[r * nbh + j];
        const float dx = st.d[r * nbh + j];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int Iv = q4_block_isum(w[p], xa, xb, xs);
          acc[p][r] = fmaf(dw[p] * dx, (float)Iv, acc[p][r]);
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < B; ++r) {
    if (r < nr) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float gv = group_sum<16>(acc[hh][r]);
        const float uv = group_sum<16>(acc[2 + hh][r]);
        const float h = silu_f(gv) * uv;
        const int nl = 8 * wv + 4 * hh + q;
        if (sub == 0) {
          hbuf[r][nl] = h;
          if (a.has_dbg && a.dbg.h) a.dbg.h[(int64_t)pairmap[r] * I + tile * 32 + nl] = h;
        }
      }
    }
  }
  __syncthreads();

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
      hv.qsum[bi] = qb.qsum;
    }
  }
}

// ---------------------------------------------------------------------------
// down + weighted combine + shared expert.  128 threads = 2 waves, a 16-lane
// group owns one output row (8 rows per workgroup); lane s reads blocks
// s, s+16, ... of the I/32 blocks of the row for each expert.
// ---------------------------------------------------------------------------
constexpr int kDownThreads = 128;
constexpr int kDownRows = kDownThreads / 16;

template <int B>
__global__ __launch_bounds__(kDownThreads) void k_moe_down(MoeArgs a) {
  __shared__ GatherLds g;
  __shared__ float pw[kMaxPairs + MMV_MAX_BATCH];

  const mmv_moe_layer &L = a.L;
  const int k = L.top_k, H = L.hidden, I = L.inter;
  const int Bk = B * k;
  const bool has_sh = L.sh_down_qs != nullptr;
  build_gather(a.ids, Bk, L.n_experts, g);
  for (int t = threadIdx.x; t < Bk + B; t += blockDim.x) {
    float v;
    if (t < Bk) v = a.weights[t];
    else v = a.shared_w ? a.shared_w[t - Bk] : 1.0f;
    pw[t] = v;
  }
  __syncthreads();

  const int nbi = I >> 5;
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int row = blockIdx.x * kDownRows + (threadIdx.x >> 4);
  const int rowc = min(row, H - 1);
  const HqView hv = hq_view(a.hq, a.P, I);
  const int U = g.U;
  const int Utot = U + (has_sh ? 1 : 0);

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;

  for (int j = sub; j < nbi; j += 16) {
    for (int u0 = 0; u0 < Utot; u0 += 4) {
      u32x4 w[4];
      float dw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = min(u0 + i, Utot - 1);
        const uint8_t *dq;
        const uint16_t *dd;
        if (u < U) {
          const int64_t eo = (int64_t)g.unique[u] * H * nbi;
          dq = L.down_qs + eo * 16; dd = L.down_d + eo;
        } else {
          dq = L.sh_down_qs; dd = L.sh_down_d;
        }
        const int64_t blk = (int64_t)rowc * nbi + j;
        w[i] = load_stream16(dq + blk * 16);
        dw[i] = f16_bits_to_f32(load_stream2(dd + blk));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = u0 + i;
        if (u < Utot) {
          const int pbeg = u < U ? g.offsets[u] : 0;
          const int pend = u < U ? g.offsets[u + 1] : B;
          for (int pi = pbeg; pi < pend; ++pi) {
            const int p = u < U ? g.pairs[pi] : Bk + pi;
            const int pb = u < U ? p / k : pi;
            const uint8_t *hc = hv.codes + (size_t)p * I + 32 * j;
            const i32x4 xa = *reinterpret_cast<const i32x4 *>(hc);
            const i32x4 xb = *reinterpret_cast<const i32x4 *>(hc + 16);
            const size_t bi = (size_t)p * nbi + j;
            const int xs = hv.qsum[bi];
            const float dh = f16_bits_to_f32(hv.ds[bi * 2]);
            const int Iv = q4_block_isum(w[i], xa, xb, xs);
            const float part = (dw[i] * dh) * (float)Iv;
            const float gw = pw[p];
#pragma unroll
            for (int b = 0; b < B; ++b)
              if (b == pb) acc[b] = fmaf(gw, part, acc[b]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float v = group_sum<16>(acc[b]);
    if (sub == 0 && row < H) a.Y[(int64_t)b * a.ldy + row] = v;
  }
}

hipError_t run_moe_experts(const mmv_moe_layer &L, const float *X, int64_t ldx, int B,
                           const int32_t *ids, const float *weights, const float *shared_w,
                           float *Y, int64_t ldy, uint8_t *hq, const mmv_moe_debug *dbg,
                           hipStream_t s) {
  MoeArgs a;
  a.L = L;
  a.X = X;
  a.ldx = ldx;
  a.ids = ids;
  a.weights = weights;
  a.shared_w = shared_w;
  a.Y = Y;
  a.ldy = ldy;
  a.hq = hq;
  const bool has_sh = L.sh_gate_qs != nullptr;
  a.P = B * L.top_k + (has_sh ? B : 0);
  a.has_dbg = dbg != nullptr;
  if (dbg) a.dbg = *dbg;
  else a.dbg = mmv_moe_debug{nullptr, nullptr, nullptr, nullptr, nullptr};

  const int slots = B * L.top_k + (has_sh ? 1 : 0);
  const int ntiles = L.inter / 32;
  const size_t lds = xstage_bytes(B, L.hidden);
  const int down_blocks = (L.hidden + kDownRows - 1) / kDownRows;
  switch (B) {
#define MMV_MOE_CASE(BB)                                                                   \
  case BB:                                                                                 \
    hipLaunchKernelGGL(k_moe_gate_up<BB>, dim3(slots * ntiles), dim3(256), lds, s, a);     \
    hipLaunchKernelGGL(k_moe_down<BB>, dim3(down_blocks), dim3(kDownThreads), 0, s, a);    \
    break;
    MMV_MOE_CASE(1) MMV_MOE_CASE(2) MMV_MOE_CASE(3) MMV_MOE_CASE(4)
    MMV_MOE_CASE(5) MMV_MOE_CASE(6) MMV_MOE_CASE(7) MMV_MOE_CASE(8)
#undef MMV_MOE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mmv
