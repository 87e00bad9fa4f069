// gemv_bf16.hip -- dense BF16 GEMV for decode, y = W x, B <= 8 rows of x.
//
// "Beating llama.cpp from Scratch on Consumer AMD" (The Optimization Passes,
// Pass 3 item 2) replaces GEMM tiles, which use their tiles poorly at M = 1,
// with a matrix-vector kernel whose vector loads stream the weights; its
// Act 6 shows that decode then sits on the memory-bandwidth wall.  On gfx950
// the same bound applies at ~8 TB/s of HBM3E, so the kernels are shaped
// around the weight stream:
//  - B = 1: one wave64 owns R whole rows; lane l reads 16-byte chunks l,
//    l+64, ... of every row (8 bf16 per 128-bit load, 1 KiB per wave
//    instruction, fully coalesced), non-temporal so x stays cached; x comes
//    through L1/L2 or is staged once per workgroup in LDS; fp32 FMAs, no
//    MFMA (a matvec); every variant sums a row in one order (chunk
//    ascending, then a fixed lane butterfly), so all give the same bits.
//  - B >= 2: 8 FMAs per weight would make the VALU the bound, so the x rows
//    become one bf16 hi/lo matrix-core operand; the weights still arrive in
//    contiguous 1 KiB wave loads and are re-laid out through LDS.  Rows
//    agree bit for bit for every B >= 2, and with B = 1 within ~1e-6.
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
      const float v = wave_sum_last(acc[r][b]);
      if (lane == 63 && row0 + r < N) Y[(int64_t)b * ldy + row0 + r] = v;
    }
  }
}

// Fixed-K variant: K = 512 * NI exactly, so every lane owns NI chunks of
// each row and all R * NI weight loads of a wave are issued before the first
// FMA.  The per-(row, b) FMA order (chunk ascending, 8 products per chunk) is
// the generic kernel's, so both variants give identical bits.
template <int B, int R, int NI, int WPB>
__global__ __launch_bounds__(WPB * 64) void k_gemv_bf16_ni(
    const uint16_t *__restrict__ W, int N, int64_t ldw, const float *__restrict__ X,
    int64_t ldx, float *__restrict__ Y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * WPB + (threadIdx.x >> 6);
  const int row0 = wave * R;
  if (row0 >= N) return;
  u32x4 w[R][NI];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint8_t *wr =
        reinterpret_cast<const uint8_t *>(W + (int64_t)min(row0 + r, N - 1) * ldw);
#pragma unroll
    for (int i = 0; i < NI; ++i) w[r][i] = load_stream16(wr + (int64_t)(lane + 64 * i) * 16);
  }
  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float *xp = X + (int64_t)b * ldx + 8 * (lane + 64 * i);
      const f32x4 xa = load_f4(xp), xb = load_f4(xp + 4);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][b] = dot8_bf16(w[r][i], xa, xb, acc[r][b]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = wave_sum_last(acc[r][b]);
      if (lane == 63 && row0 + r < N) Y[(int64_t)b * ldy + row0 + r] = v;
    }
  }
}

// LDS-x variant for K = 512 * NI and B rows of x: a workgroup of WPB waves
// (R rows each) requests x (once for the workgroup instead of once per
// wave), then every weight chunk of its rows; x goes to LDS while the
// weights are in flight, and the FMAs read it from there, each x chunk once
// for the R rows.  x is staged in slabs of SL chunks (B * SL * 2 KiB of LDS),
// slab after slab when K is longer, the next slab's loads in flight while
// the current one is used.  Every (row, b) sum has the order of
// k_gemv_bf16_ni (chunk ascending, 8 products per chunk, then the lanes),
// whatever B, R, WPB and SL: all give the bits of the B = 1 kernel, row by
// row.
template <int B, int NI, int WPB, int R, int SL>
__global__ __launch_bounds__(WPB * 64) void k_gemv_bf16_xl(
    const uint16_t *__restrict__ W, int N, int64_t ldw, const float *__restrict__ X,
    int64_t ldx, float *__restrict__ Y, int64_t ldy) {
  extern __shared__ __align__(16) float xs[];  // [B][SL * 512]
  constexpr int NT = WPB * 64;
  constexpr int NSL = (NI + SL - 1) / SL;     // slabs
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * WPB + (threadIdx.x >> 6)) * R;

  // float4 task t of slab sl: row b = t / (nc * 128), chunk c0 + (t % ...)
  auto slab_load = [&](int sl, f32x4 (&xv)[(B * SL * 128 + NT - 1) / NT]) {
    const int c0 = sl * SL, nc = min(SL, NI - c0), tot = B * nc * 128;
#pragma unroll
    for (int m = 0; m < (B * SL * 128 + NT - 1) / NT; ++m) {
      const int t = min((int)threadIdx.x + NT * m, tot - 1);
      const int b = t / (nc * 128), q = t - b * nc * 128;
      xv[m] = load_f4(X + (int64_t)b * ldx + 4 * (c0 * 128 + q));
    }
  };
  auto slab_store = [&](int sl, const f32x4 (&xv)[(B * SL * 128 + NT - 1) / NT]) {
    const int nc = min(SL, NI - sl * SL), tot = B * nc * 128;
#pragma unroll
    for (int m = 0; m < (B * SL * 128 + NT - 1) / NT; ++m) {
      const int t = (int)threadIdx.x + NT * m;
      if (t < tot) {
        const int b = t / (nc * 128), q = t - b * nc * 128;
        *reinterpret_cast<f32x4 *>(&xs[b * SL * 512 + 4 * q]) = xv[m];
      }
    }
  };

  f32x4 xv[(B * SL * 128 + NT - 1) / NT];
  slab_load(0, xv);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 w[R][NI];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint8_t *wr =
        reinterpret_cast<const uint8_t *>(W + (int64_t)min(row0 + r, N - 1) * ldw);
#pragma unroll
    for (int i = 0; i < NI; ++i) w[r][i] = load_stream16(wr + (int64_t)(lane + 64 * i) * 16);
  }
  __builtin_amdgcn_sched_barrier(0);
  float acc[R * B];
#pragma unroll
  for (int j = 0; j < R * B; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    if (sl > 0) __syncthreads();  // the previous slab is consumed
    slab_store(sl, xv);
    __syncthreads();
    if (sl + 1 < NSL) slab_load(sl + 1, xv);  // in flight while this slab is used
#pragma unroll
    for (int i = sl * SL; i < (sl + 1) * SL && i < NI; ++i) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float *xp = xs + b * SL * 512 + 8 * (lane + 64 * (i - sl * SL));
        const f32x4 xa = *reinterpret_cast<const f32x4 *>(xp);
        const f32x4 xb = *reinterpret_cast<const f32x4 *>(xp + 4);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r * B + b] = dot8_bf16(w[r][i], xa, xb, acc[r * B + b]);
      }
    }
  }
  gsum_last_n<64>(acc);
  if (lane == 63) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (row0 + r < N)
#pragma unroll
        for (int b = 0; b < B; ++b) Y[(int64_t)b * ldy + row0 + r] = acc[r * B + b];
  }
}

// B >= 2 when K % 512 != 0: v_mfma_f32_16x16x32_bf16 takes a
// 16-row x 32-k tile of W (one 128-bit load per lane: row l%16, k 8*(l/16)..)
// against x^T (column l%16 = activation row b, zero for b >= B).  fp32 x is
// split exactly into bf16 hi + lo (x - hi is exact in fp32; lo keeps the next
// 8 bits), two MFMAs per step, so products keep ~2^-17 relative accuracy.
// A workgroup owns one 16-row tile; its KS waves take interleaved k-steps
// (wave w: steps w, w+KS, ...), so the workgroup streams each row
// contiguously, and the KS partial tiles are summed in LDS in wave order.
// Column b of the result depends only on x row b: rows agree bit for bit for
// every B >= 2.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split_bf16(f32x4 a, f32x4 b, bf16x8 &hi, bf16x8 &lo) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)v[j];
    hi[j] = h;
    lo[j] = (__bf16)(v[j] - (float)h);
  }
}

template <int B, int KS, int U>
__global__ __launch_bounds__(KS * 64) void k_gemv_bf16_mfma(
    const uint16_t *__restrict__ W, int N, int K, int64_t ldw, const float *__restrict__ X,
    int64_t ldx, float *__restrict__ Y, int64_t ldy) {
  __shared__ float part[KS][16][B];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int r = lane & 15, g = lane >> 4;
  const bool colv = r < B;  // B operand column = activation row
  const uint8_t *wr = reinterpret_cast<const uint8_t *>(W + (int64_t)min(n0 + r, N - 1) * ldw);
  const float *xr = X + (int64_t)min(r, B - 1) * ldx;
  const int nsteps = (K + 31) >> 5;
  const int nj = w < nsteps ? (nsteps - w + KS - 1) / KS : 0;  // this wave's steps
  typedef float f32x4m __attribute__((ext_vector_type(4)));
  f32x4m acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // Chunks of U steps with no branches inside: a step past the wave's last
  // one re-reads that last step (same lines) with its x zeroed, and k >= K
  // reads are clamped in bounds and zeroed; x is loaded before W so that,
  // loads completing in order, step u waits only for its own loads.
  for (int j0 = 0; j0 < nj; j0 += U) {
    f32x4 xa[U], xb[U];
    u32x4 a[U];
    int kk[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(j0 + u, nj - 1);
      const int k = (w + KS * j) * 32 + 8 * g;
      ok[u] = colv && (j0 + u < nj) && (k < K);
      kk[u] = min(k, K - 8);
      xa[u] = load_f4(xr + kk[u]);
      xb[u] = load_f4(xr + kk[u] + 4);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = load_stream16(wr + 2 * (int64_t)kk[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      bf16x8 hi, lo;
      split_bf16(ok[u] ? xa[u] : z, ok[u] ? xb[u] : z, hi, lo);
      const bf16x8 av = __builtin_bit_cast(bf16x8, a[u]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, lo, acc, 0, 0, 0);
    }
  }
  // lane holds rows 4g..4g+3 of column r
  if (colv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) part[w][4 * g + i][r] = acc[i];
  }
  __syncthreads();
  if (threadIdx.x < 16 * B) {
    const int row = threadIdx.x / B, b = threadIdx.x - row * B;
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < KS; ++q) v += part[q][row][b];
    if (n0 + row < N) Y[(int64_t)b * ldy + n0 + row] = v;
  }
}

// x as one matrix-core operand for B >= 2: 16 columns made from the B rows
// of x, column c < 8 holding bf16(x_c) (round to nearest even) and column
// 8 + c the rounded remainder bf16(x_c - bf16(x_c)) (the subtraction is
// exact in fp32), zero for c >= B; y[n][c] = D[n][c] + D[n][c + 8] keeps
// ~2^-17 relative accuracy per product with one MFMA per step.  Each lane
// loads only half of its 8 x values and takes the other half from the lane
// 8 places along its 16-lane row (DPP row_ror:8).
constexpr int kDppRowRor8 = 0x128;

typedef float f32x4v __attribute__((ext_vector_type(4)));

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16_pair_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2v));
}

// 8 consecutive x values -> this lane's 8 B-operand entries (hi or lo half)
__device__ __forceinline__ bf16x8 x_operand(f32x4 p, f32x4 q, bool lo, uint32_t keep) {
  const float v[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = bf16_pair_bits(v[2 * i], v[2 * i + 1]);
    const uint32_t l = bf16_pair_bits(v[2 * i] - bf16_lo(h), v[2 * i + 1] - bf16_hi(h));
    out[i] = (lo ? l : h) & keep;
  }
  return __builtin_bit_cast(bf16x8, out);
}

// B >= 2 through LDS: the workgroup streams RT rows in chunks of 1 KiB per
// row with contiguous 1 KiB wave loads (the pattern HBM serves best; loads
// in the operand layout itself, 16 rows x 64 B per instruction, ran ~30%
// slower), stores each chunk to LDS, and reads it back in the operand
// layout of v_mfma_f32_16x16x32_bf16 (A = 16 weight rows x 32 k, lane l:
// row l % 16, k 8 * (l / 16) ..).  Chunk i + PD is in flight while chunk i
// is multiplied.  The NW waves split each chunk's 16 k-steps (wave w: steps
// w, w + NW, ...) and make their own x operands for every row tile of the
// workgroup; partial tiles are summed in LDS in wave order at the end, so a
// row's bits depend on NW only (not on RT, PD, TH or B).  TH = 8: tiles of
// 8 rows (operand rows 8..15 repeat rows 0..7).  NCH > 0 fixes the chunk
// count (K = 512 NCH) and unrolls every chunk: a loop would carry the
// prefetch registers around its back edge, and the copies that makes wait
// for the loads still filling them.  Needs K % 512 == 0.
constexpr int kMlChunk = 1024;             // bytes of a row per chunk
constexpr int kMlPitch = kMlChunk + 16;    // LDS row pitch: 16-B skew between rows

template <int B, int RT, int NW>
constexpr size_t ml_lds_bytes() {
  return (size_t)2 * RT * kMlPitch + (size_t)NW * RT * B * 4;
}

template <int B, int RT, int NW, int PD, int TH, int NCH = 0>
__global__ __launch_bounds__(NW * 64) void k_gemv_bf16_ml(
    const uint16_t *__restrict__ W, int N, int K, int64_t ldw, const float *__restrict__ X,
    int64_t ldx, float *__restrict__ Y, int64_t ldy) {
  constexpr int LPC = RT / NW;    // weight loads per lane per chunk (one row each)
  constexpr int SPW = 16 / NW;    // k-steps per wave per chunk
  constexpr int TILES = (RT + 15) / 16;
  static_assert(RT % NW == 0 && 16 % NW == 0 && (TH == 16 || RT == 8), "shape");
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t *abuf = smem;                                                  // [2][RT][pitch]
  float *part = reinterpret_cast<float *>(smem + (size_t)2 * RT * kMlPitch);  // [NW][RT][B]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4, c = n & 7;
  const bool lo = n >= 8;
  const int rb = blockIdx.x * RT;
  const int nch = NCH ? NCH : K >> 9;
  const uint8_t *wsrc[LPC];
#pragma unroll
  for (int j = 0; j < LPC; ++j)
    wsrc[j] = reinterpret_cast<const uint8_t *>(W + (int64_t)min(rb + w + NW * j, N - 1) * ldw) +
              16 * lane;
  const float *xr = X + (int64_t)min(c, B - 1) * ldx + (lo ? 4 : 0) + 8 * g + 32 * w;
  const uint32_t keep = c < B ? 0xFFFFFFFFu : 0u;

  u32x4 wreg[PD][LPC];
  f32x4 xreg[PD][SPW];
  // x first, then weights: loads complete in order, so chunk i's x and
  // weights arrive without waiting for later chunks
  auto issue = [&](int ch, u32x4(&wr)[LPC], f32x4(&xg)[SPW]) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) xg[s] = load_f4(xr + 512 * ch + 32 * NW * s);
#pragma unroll
    for (int j = 0; j < LPC; ++j) wr[j] = load_stream16(wsrc[j] + (int64_t)kMlChunk * ch);
  };
#pragma unroll
  for (int p = 0; p < PD; ++p)
    if (p < nch) issue(p, wreg[p], xreg[p]);

  f32x4v acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  // NCH > 0: every chunk unrolled, so no register is carried around a loop
  // (a copy of a register that a load is still filling would wait for it);
  // NCH == 0: a loop over the run-time chunk count
  constexpr int kChunkUnroll = NCH > 0 ? NCH : 1;
#pragma unroll kChunkUnroll
  for (int i0 = 0; i0 < (NCH ? NCH : nch); i0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int i = i0 + p;
      if (i < nch) {
        uint8_t *buf = abuf + (size_t)(i & 1) * RT * kMlPitch;
#pragma unroll
        for (int j = 0; j < LPC; ++j)
          *reinterpret_cast<u32x4 *>(buf + (w + NW * j) * kMlPitch + 16 * lane) = wreg[p][j];
        bf16x8 xb[SPW];
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          f32x4 o;
          o.x = dpp_f32<kDppRowRor8>(xreg[p][s].x);
          o.y = dpp_f32<kDppRowRor8>(xreg[p][s].y);
          o.z = dpp_f32<kDppRowRor8>(xreg[p][s].z);
          o.w = dpp_f32<kDppRowRor8>(xreg[p][s].w);
          xb[s] = x_operand(lo ? o : xreg[p][s], lo ? xreg[p][s] : o, lo, keep);
        }
        __syncthreads();
        if (i + PD < nch) issue(i + PD, wreg[p], xreg[p]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          const int st = w + NW * s;
#pragma unroll
          for (int t = 0; t < TILES; ++t) {
            const int row = t * 16 + (TH == 16 ? n : c);
            const u32x4 av = *reinterpret_cast<const u32x4 *>(buf + row * kMlPitch + 64 * st + 16 * g);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), xb[s],
                                                             acc[t], 0, 0, 0);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = acc[t][i] + dpp_f32<kDppRowRor8>(acc[t][i]);
      const int m = 4 * g + i;
      if (!lo && c < B && m < TH) part[(w * RT + t * 16 + m) * B + c] = v;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < RT * B; idx += NW * 64) {
    const int r = idx / B, cc = idx - r * B;
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < NW; ++q) v += part[(q * RT + r) * B + cc];
    if (rb + r < N) Y[(int64_t)cc * ldy + rb + r] = v;
  }
}

namespace {

struct Bf16Args {
  const uint16_t *W;
  int N, K;
  int64_t ldw;
  const float *X;
  int64_t ldx;
  float *Y;
  int64_t ldy;
  hipStream_t s;
};

template <int B, int R, int U>
hipError_t launch_generic(const Bf16Args &a) {
  const int waves = (a.N + R - 1) / R;
  hipLaunchKernelGGL((k_gemv_bf16<B, R, U>), dim3((waves + 3) / 4), dim3(256), 0, a.s, a.W,
                     a.N, a.K, a.ldw, a.X, a.ldx, a.Y, a.ldy);
  return hipGetLastError();
}

template <int B, int R, int NI, int WPB>
hipError_t launch_ni(const Bf16Args &a) {
  const int waves = (a.N + R - 1) / R;
  hipLaunchKernelGGL((k_gemv_bf16_ni<B, R, NI, WPB>), dim3((waves + WPB - 1) / WPB),
                     dim3(WPB * 64), 0, a.s, a.W, a.N, a.ldw, a.X, a.ldx, a.Y, a.ldy);
  return hipGetLastError();
}

template <int B, int NI>
hipError_t dispatch_ni(const Bf16Args &a, int R, int WPB) {
  // all R * NI weight loads of a lane sit in registers (4 VGPRs each):
  // only variants with R * NI <= 24 exist
  if constexpr (NI * 4 <= 24 && B <= 2) {
    if (R >= 4) return WPB == 1 ? launch_ni<B, 4, NI, 1>(a) : launch_ni<B, 4, NI, 4>(a);
  }
  if constexpr (NI * 2 <= 24) {
    if (R >= 2) return WPB == 1 ? launch_ni<B, 2, NI, 1>(a) : launch_ni<B, 2, NI, 4>(a);
  }
  return WPB == 1 ? launch_ni<B, 1, NI, 1>(a) : launch_ni<B, 1, NI, 4>(a);
}

template <int B, int KS, int U>
hipError_t launch_mfma(const Bf16Args &a) {
  hipLaunchKernelGGL((k_gemv_bf16_mfma<B, KS, U>), dim3((a.N + 15) / 16), dim3(KS * 64), 0,
                     a.s, a.W, a.N, a.K, a.ldw, a.X, a.ldx, a.Y, a.ldy);
  return hipGetLastError();
}

template <int B, int RT, int NW, int PD, int TH, int NCH = 0>
hipError_t launch_ml(const Bf16Args &a) {
  constexpr size_t lds = ml_lds_bytes<B, RT, NW>();
  if (lds > 65536) {
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_gemv_bf16_ml<B, RT, NW, PD, TH, NCH>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (raised != hipSuccess) return raised;
  }
  hipLaunchKernelGGL((k_gemv_bf16_ml<B, RT, NW, PD, TH, NCH>), dim3((a.N + RT - 1) / RT),
                     dim3(NW * 64), lds, a.s, a.W, a.N, a.K, a.ldw, a.X, a.ldx, a.Y, a.ldy);
  return hipGetLastError();
}

template <int B, int RT, int NW, int PD, int TH>
hipError_t launch_mlu(const Bf16Args &a) {
  switch (a.K >> 9) {
    case 4: return launch_ml<B, RT, NW, PD, TH, 4>(a);
    case 5: return launch_ml<B, RT, NW, PD, TH, 5>(a);
    case 8: return launch_ml<B, RT, NW, PD, TH, 8>(a);
    case 19: return launch_ml<B, RT, NW, PD, TH, 19>(a);
  }
  return launch_ml<B, RT, NW, PD, TH>(a);
}

// B >= 2 and K % 512 == 0.  The MMV_PATH_BF16_ML switch (tests) = 10000 * RT
// + 1000 * NW + 100 * PD + TH, + 1000000 for the chunk loop instead of the
// unrolled chunks.  Default: 16-row workgroups of 8 waves, two chunks in
// flight (2560 x 2560 / 19456 x 2560 / 2560 x 9728 at B = 8: 6.0 / 21 /
// 15.7 us against 8.2 / 26 / 27.7 us for FMAs with x in LDS or the operand-
// layout loads).
template <int B>
hipError_t dispatch_ml(const Bf16Args &a, int knob) {
  switch (knob) {
    case 0: return launch_mlu<B, 16, 8, 2, 16>(a);
    case 1168216: return launch_ml<B, 16, 8, 2, 16>(a);
    case 1328216: return launch_ml<B, 32, 8, 2, 16>(a);
    case 1168316: return launch_ml<B, 16, 8, 3, 16>(a);
    case 1088208: return launch_ml<B, 8, 8, 2, 8>(a);
    case 1164216: return launch_ml<B, 16, 4, 2, 16>(a);
  }
  return launch_mlu<B, 16, 8, 2, 16>(a);  // an unknown shape code: the default
}

// slab length: x of B rows in at most 80 KiB of LDS (SL chunks of 512)
template <int B, int NI>
constexpr int xl_slab() { return cmin(NI, 40 / B); }

template <int B, int NI, int WPB, int R>
hipError_t launch_xl(const Bf16Args &a) {
  constexpr int RPB = WPB * R, SL = xl_slab<B, NI>();
  const size_t lds = (size_t)B * SL * 512 * 4;
  hipLaunchKernelGGL((k_gemv_bf16_xl<B, NI, WPB, R, SL>), dim3((a.N + RPB - 1) / RPB),
                     dim3(WPB * 64), lds, a.s, a.W, a.N, a.ldw, a.X, a.ldx, a.Y, a.ldy);
  return hipGetLastError();
}

template <int NI>
hipError_t dispatch_xl(const Bf16Args &a, int WPB) {
  if (WPB == 10) return launch_xl<1, NI, 10, 1>(a);
  if (WPB == 5) return launch_xl<1, NI, 5, 1>(a);
  if (WPB >= 16) return launch_xl<1, NI, 16, 1>(a);
  if (WPB >= 8) return launch_xl<1, NI, 8, 1>(a);
  if (WPB >= 4) return launch_xl<1, NI, 4, 1>(a);
  return launch_xl<1, NI, 2, 1>(a);
}

// waves per workgroup (one row each) for N rows at B = 1 when rows are few:
// of 10, 8, 5 and 4, the one whose rounds of one workgroup per CU
// leave the fewest wave slots empty; ties go to the larger workgroup
inline int xl_waves(int N) {
  const int64_t cus = cu_count();
  int best = 10;
  int64_t best_idle = -1;
  for (int w : {10, 8, 5, 4}) {
    const int64_t wgs = (N + w - 1) / w, rounds = (wgs + cus - 1) / cus;
    const int64_t idle = rounds * cus * w - N;
    if (best_idle < 0 || idle < best_idle) best = w, best_idle = idle;
  }
  return best;
}

template <int B>
hipError_t dispatch_b(const Bf16Args &a) {
  if constexpr (B >= 2) {
    if (a.K % 512 == 0) return dispatch_ml<B>(a, path_switch(MMV_PATH_BF16_ML));
    // other K: operand-layout loads, KS waves per 16-row tile
    const int kw = path_switch(MMV_PATH_BF16_WAVES);
    const int KS = kw ? kw : 8;
    if (KS >= 16) return launch_mfma<B, 16, 8>(a);
    if (KS >= 8) return launch_mfma<B, 8, 8>(a);
    return launch_mfma<B, 4, 8>(a);
  } else {
    const int kr = path_switch(MMV_PATH_BF16_ROWS), kw = path_switch(MMV_PATH_BF16_WAVES);
    const int kx = path_switch(MMV_PATH_BF16_XL);
    if (a.K % 512 == 0) {
      // x staged once per workgroup in LDS.  Many rows (19456 x 2560): 8
      // waves per workgroup.  Fewer rows: a workgroup size that spreads the
      // rows evenly over the CUs (2560 x 9728: 256 workgroups of 10 waves,
      // 9.9 us, against 10.9 us for 640 of 4, whose last round leaves CUs
      // idle; 2560 x 2560: 4.25 against 4.31 us for the per-wave kernel)
      const int NI = a.K / 512;
      const int xl = kx != 0 ? kx : (NI >= 4 && a.N >= 8192 ? 8 : (NI >= 4 ? xl_waves(a.N) : -1));
      if (xl > 0) {
        switch (NI) {
          case 4: return dispatch_xl<4>(a, xl);
          case 5: return dispatch_xl<5>(a, xl);
          case 8: return dispatch_xl<8>(a, xl);
          case 16: return dispatch_xl<16>(a, xl);
          case 19: return dispatch_xl<19>(a, xl);
          default: break;
        }
      }
    }
    if (a.K % 512 == 0) {
      const int NI = a.K / 512;
      // enough rows per wave that a wave streams >= ~8 KiB; one-wave
      // workgroups unless the grid is very large
      const int R = kr ? kr : (NI >= 8 ? 1 : (a.N >= 4096 ? 2 : 1));
      const int waves = (a.N + R - 1) / R;
      const int WPB = kw ? kw : (waves >= 16384 ? 4 : 1);
      switch (NI) {
        case 1: return dispatch_ni<B, 1>(a, R, WPB);
        case 2: return dispatch_ni<B, 2>(a, R, WPB);
        case 4: return dispatch_ni<B, 4>(a, R, WPB);
        case 5: return dispatch_ni<B, 5>(a, R, WPB);
        case 8: return dispatch_ni<B, 8>(a, R, WPB);
        case 19: return dispatch_ni<B, 19>(a, R, WPB);
        default: break;
      }
    }
    if (a.N >= 8192) return launch_generic<B, 4, 4>(a);
    if (a.N >= 4096) return launch_generic<B, 2, 4>(a);
    return launch_generic<B, 1, 4>(a);
  }
}

}  // namespace

hipError_t run_gemv_bf16(const uint16_t *W, int N, int K, int64_t ldw,
                         const float *X, int64_t ldx, int B, float *Y, int64_t ldy,
                         hipStream_t s) {
  const Bf16Args a{W, N, K, ldw, X, ldx, Y, ldy, s};
  switch (B) {
    case 1: return dispatch_b<1>(a);
    case 2: return dispatch_b<2>(a);
    case 3: return dispatch_b<3>(a);
    case 4: return dispatch_b<4>(a);
    case 5: return dispatch_b<5>(a);
    case 6: return dispatch_b<6>(a);
    case 7: return dispatch_b<7>(a);
    case 8: return dispatch_b<8>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace mmv
