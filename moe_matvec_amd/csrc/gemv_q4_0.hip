// gemv_q4_0.hip -- Q4_0 weights x Q8_1 activations (v_dot4 and int8
// matrix-core kernels), Q4_0 weights x fp32 activations (W4A16: v_dot2 and
// bf16 matrix-core kernels), and the standalone activation quantizer.
//
// "Fourteen hours to 100 tokens per second" (The trace that changed
// everything) lists the dense Q4_0 matvecs and quantize_q8_1 as separate
// kernel classes; "Eight levers that worked" gives the down projection
// (K <= 512) four rows per wave with 16 lanes per row.  On gfx950:
//  - a row is owned by a lane group of G lanes (G = 16 for K <= 512, up to 64
//    for long rows); lane s of the group reads Q4_0 blocks s, s+G, ... of the
//    row: one 128-bit code load + one fp16 scale per block, coalesced across
//    the group (G*16 contiguous bytes per row per instruction);
//  - the workgroup first issues its first weight loads, then stages x as
//    Q8_1 in LDS (quantizing fp32 x with the shared routine, or copying a
//    Q8_1 buffer) while those loads are in flight;
//  - per block: nibble unpack with two masks, 8 v_dot4 on int8, exact int32
//    sum, then one fp32 scale and fma per activation row;
//  - each x block read from LDS is reused for the RP rows a lane owns;
//  - group partials are combined by a fixed xor butterfly; the per-row
//    arithmetic of the v_dot4 kernels is the same for every B and every
//    workgroup shape (4 or 8 waves, any rows per lane group), so their rows
//    of a batched call match single-row calls bit for bit; the matrix-core
//    kernels below sum in their own orders.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "q4_0.hpp"
#include "q8_1.hpp"

namespace mmv {

// ---- standalone quantize_q8_1 ------------------------------------------
// 8 lanes per block; a workgroup of 256 threads quantizes 32 blocks.
__global__ __launch_bounds__(256) void k_quantize_q8_1(const float *__restrict__ X, int K,
                                                       int64_t ldx, int B, uint8_t *__restrict__ Xq) {
  const int nb = K >> 5;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)B * nb * 8;
  // keep whole 8-lane groups active: total is a multiple of 8
  if (t >= total) return;
  const int b = (int)(t / (nb * 8));
  const int rem = (int)(t - (int64_t)b * nb * 8);
  const int j = rem >> 3, s = rem & 7;
  const f32x4 v = load_f4(X + (int64_t)b * ldx + 32 * j + 4 * s);
  const Q8Block q = q8_1_quantize8(v);
  *reinterpret_cast<uint32_t *>(Xq + (size_t)b * K + 32 * j + 4 * s) = q.codes;
  if (s == 0) {
    uint16_t *ds = reinterpret_cast<uint16_t *>(Xq + (size_t)B * K);
    ds[((size_t)b * nb + j) * 2 + 0] = q.d16;
    ds[((size_t)b * nb + j) * 2 + 1] = q.s16;
  }
}

hipError_t run_quantize_q8_1(const float *X, int K, int64_t ldx, int B, uint8_t *Xq,
                             hipStream_t s) {
  const int64_t total = (int64_t)B * (K / 32) * 8;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(k_quantize_q8_1, dim3(blocks), dim3(256), 0, s, X, K, ldx, B, Xq);
  return hipGetLastError();
}

// ---- Q4_0 GEMV -----------------------------------------------------------
// B activation rows; G lanes per weight row; RP rows per lane group.  A wave
// covers RP * (64/G) rows, a 256-thread workgroup 4x that ("row group").
// The grid is at most a few workgroups per CU; each stages x once and walks
// row groups blockIdx.x, blockIdx.x + gridDim.x, ...
// activations preloaded in registers: 8 float4 per thread covers B*K <= 8192
constexpr int XPRE_MAXT = 8;

template <int B, int G, int RP>
__global__ __launch_bounds__(256) void k_gemv_q4_0(
    const uint8_t *__restrict__ qs, const uint16_t *__restrict__ dw, int N, int K,
    const float *__restrict__ X, int64_t ldx, const uint8_t *__restrict__ Xq,
    float *__restrict__ Y, int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int RPP = 64 / G;
  constexpr int ROWS_WAVE = RP * RPP;
  constexpr int ROWS_WG = 4 * ROWS_WAVE;
  const int nb = K >> 5;
  const int lane = threadIdx.x & 63;
  const int sub = lane % G, grp = lane / G;
  const int wv = threadIdx.x >> 6;
  const int ngroups = (N + ROWS_WG - 1) / ROWS_WG;
  int gi = blockIdx.x;

  // fp32 activations are loaded before the first weight blocks (loads
  // complete in issue order), so quantizing them does not wait for HBM
  constexpr int MAXT = XPRE_MAXT;
  XPre<MAXT> xp;
  const bool pre = X && (B * K <= MAXT * 4 * 256);
  if (pre) xpre_load(X, ldx, nullptr, B, K, xp);

  // first weight blocks of the first row group in flight before staging x
  u32x4 w0[RP];
  float d0[RP];
  {
    const int rbase = gi * ROWS_WG + wv * ROWS_WAVE + grp;
    const int j0 = sub < nb ? sub : 0;
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      const int64_t blk = (int64_t)min(rbase + p * RPP, N - 1) * nb + j0;
      w0[p] = load_stream16(qs + blk * 16);
      d0[p] = f16_bits_to_f32(load_stream2(dw + blk));
    }
  }

  const XStage st = xstage_at(smem, B, K);
  if (pre) xpre_quantize(xp, B, K, st);
  else if (X) stage_quantize(X, ldx, nullptr, B, K, st);
  else stage_copy_q8(Xq, B, B, K, st);
  __syncthreads();

  bool first = true;
  for (; gi < ngroups; gi += gridDim.x) {
    const int rbase = gi * ROWS_WG + wv * ROWS_WAVE + grp;  // row of pass p: + p * RPP
    int rowc[RP];
#pragma unroll
    for (int p = 0; p < RP; ++p) rowc[p] = min(rbase + p * RPP, N - 1);
    float acc[RP][B];
#pragma unroll
    for (int p = 0; p < RP; ++p)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[p][b] = 0.0f;

    for (int j = sub; j < nb; j += G) {
      u32x4 w[RP];
      float dwf[RP];
      if (first && j == sub) {
#pragma unroll
        for (int p = 0; p < RP; ++p) { w[p] = w0[p]; dwf[p] = d0[p]; }
      } else {
#pragma unroll
        for (int p = 0; p < RP; ++p) {
          const int64_t blk = (int64_t)rowc[p] * nb + j;
          w[p] = load_stream16(qs + blk * 16);
          dwf[p] = f16_bits_to_f32(load_stream2(dw + blk));
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const i32x4 xa = xstage_lo(st, b, K, j);
        const i32x4 xb = xstage_hi(st, b, K, j);
        const int xs = st.qsum[b * nb + j];
        const float dx = st.d[b * nb + j];
#pragma unroll
        for (int p = 0; p < RP; ++p) {
          const int I = q4_block_isum(w[p], xa, xb, xs);
          acc[p][b] = fmaf(dwf[p] * dx, (float)I, acc[p][b]);
        }
      }
    }

#pragma unroll
    for (int p = 0; p < RP; ++p) {
      const int row = rbase + p * RPP;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float v = gsum_last<G>(acc[p][b]);
        if (sub == G - 1 && row < N) Y[(int64_t)b * ldy + row] = v;
      }
    }
    first = false;
  }
}

// Whole-row variant: K = 32 * G * T, or with RAG any K <= 32 * G * T, so
// each lane owns at most T blocks of each of its RP rows (blocks sub + G t;
// past a ragged row's last block the load repeats that block, in bounds,
// and the step is skipped), and a workgroup of NW waves owns one group of
// NW * RP * (64 / G) consecutive rows.  The activation
// loads are issued first, then all RP * T weight loads of the group; the
// activation is quantized into LDS while the weights are in flight (loads
// complete in issue order).  Per-row arithmetic order is the same as in
// k_gemv_q4_0: block j's integer sum scaled by d_w * d_x and accumulated
// over j = sub, sub + G, ..., then a G-lane sum.
template <int B, int G, int RP, int T, bool FROM_X, bool RAG, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_gemv_q4_0_t(
    const uint8_t *__restrict__ qs, const uint16_t *__restrict__ dw, int N, int Kr,
    const float *__restrict__ X, int64_t ldx, const uint8_t *__restrict__ Xq,
    float *__restrict__ Y, int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int RPP = 64 / G;
  constexpr int ROWS_WAVE = RP * RPP;
  constexpr int NT = 64 * NW;  // threads per workgroup
  constexpr int ROWS_WG = NW * ROWS_WAVE;
  // RAG: K <= 32 G T at run time (the launcher checks it); else exactly 32 G T
  const int K = RAG ? Kr : 32 * G * T, nb = K >> 5;
  const int lane = threadIdx.x & 63;
  const int sub = lane % G, grp = lane / G;
  const int wv = threadIdx.x >> 6;

  // first pass of the activation loads, ahead of the weights: 8 B G T / NT
  // float4 tasks (or 2 B G T / NT 16-byte code tasks) per thread in all
  // (one row of a ragged long row: all of x in the first pass, 8 G T / NT
  // tasks, where the registers allow it, so that no L2 round trip of x follows the
  // weight loads)
  constexpr int MAXT = (RAG && B == 1 && T <= 7) ? cmax(1, 8 * G * T / NT)
                                                 : cmin(kStageMaxT, cmax(1, 8 * B * G * T / NT));
  constexpr int MAXC = cmin(kStageMaxC, cmax(1, 2 * B * G * T / NT));
  XPre<FROM_X ? MAXT : 1> xp;
  XqPre<FROM_X ? 1 : MAXC> qp;
  if constexpr (FROM_X) xpre_load(X, ldx, nullptr, B, K, xp, 0, NT);
  else xq_pre_load(Xq, B, B, K, qp, 0, NT);
  __builtin_amdgcn_sched_barrier(0);  // keep the weight loads behind these

  const int rbase = blockIdx.x * ROWS_WG + wv * ROWS_WAVE + grp;
  u32x4 w[RP][T];
  float d[RP][T];
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int64_t rowblk = (int64_t)min(rbase + p * RPP, N - 1) * nb;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t blk = rowblk + min(sub + G * t, nb - 1);
      w[p][t] = load_stream16(qs + blk * 16);
      d[p][t] = f16_bits_to_f32(load_stream2(dw + blk));
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // all weight loads issued before any wait

  const XStage st = xstage_at(smem, B, K);
  if constexpr (FROM_X) {
    xpre_quantize(xp, B, K, st, 0, NT);
    stage_quantize(X, ldx, nullptr, B, K, st, MAXT * NT, NT);
  } else {
    xq_pre_store(qp, B, K, st, 0, NT);
    stage_copy_q8(Xq, B, B, K, st, MAXC * NT, NT);
  }
  __syncthreads();

  float acc[RP][B];
#pragma unroll
  for (int p = 0; p < RP; ++p)
#pragma unroll
    for (int r = 0; r < B; ++r) acc[p][r] = 0.0f;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int j = sub + G * t;
    if (j < nb) {  // false only in the last step of a ragged row
#pragma unroll
      for (int r = 0; r < B; ++r) {
        const i32x4 xa = xstage_lo(st, r, K, j);
        const i32x4 xb = xstage_hi(st, r, K, j);
        const int xs = st.qsum[r * nb + j];
        const float dx = st.d[r * nb + j];
#pragma unroll
        for (int p = 0; p < RP; ++p) {
          const int I = q4_block_isum(w[p][t], xa, xb, xs);
          acc[p][r] = fmaf(d[p][t] * dx, (float)I, acc[p][r]);
        }
      }
    }
  }
  float (&flat)[RP * B] = *reinterpret_cast<float(*)[RP * B]>(&acc[0][0]);
  gsum_last_n<G>(flat);
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int row = rbase + p * RPP;
#pragma unroll
    for (int r = 0; r < B; ++r)
      if (sub == G - 1 && row < N) Y[(int64_t)r * ldy + row] = acc[p][r];
  }
}

// ---- W4A16: Q4_0 weights x fp32 activations, no Q8_1 step ---------------
// "Beating llama.cpp from Scratch on Consumer AMD" ("BF16 vs Quantization")
// names W4A16 INT4 weights with on-the-fly dequantization as the variant
// that trades integer unpacking for activation precision.  Same row layout
// as k_gemv_q4_0_t (G lanes per row, RP rows per lane group, weight loads
// issued after the first activation loads).  x is split into bf16 high and
// low parts (x - hi is exact in fp32; lo keeps the next 8 bits, so hi + lo
// is x to 2^-17 relative) and staged in LDS block-transposed: 16 bytes per
// (b, q, j), q = 0..7 within a block, holding hi(x0 x1), hi(x2 x3),
// lo(x0 x1), lo(x2 x3) of positions 4q..4q+3, so lanes reading consecutive
// blocks read consecutive 16-byte words.  Each block's -136 sum_i (hi + lo)
// is staged beside it.  A code becomes bf16 128 + c by one v_perm per two
// codes (exponent byte 0x43 above the code byte), and v_dot2c_f32_bf16 takes
// two codes times two x parts per instruction (products exact in fp32).  Per
// block: S = -136 sum (hi + lo), then S += (128 + c) . hi and (128 + c) . lo
// (k ascending through the low then the high nibbles), value d_w * S =
// d_w sum (c - 8)(hi + lo).  Every (row, b) sum runs over the lane's blocks
// j = sub, sub + G, ... in ascending order, then the G-lane sum: one order
// for every B and in both kernels below (same G), so rows are bit-identical
// whatever the batch and the kernel.
constexpr int kF32Pass = 8;  // float4 staging tasks per thread per pass

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {  // round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// row of task t (0 <= t < B * per_row) of a row-major [B][per_row] array:
// no division for one or two rows
template <int B>
__device__ __forceinline__ int task_row(int t, int per_row) {
  if constexpr (B == 1) return 0;
  else if constexpr (B == 2) return t >= per_row ? 1 : 0;
  else return t / per_row;
}

// one float4 of x (task t of the [B][K/4] row-major x) to the staged layout;
// the block's sum is formed by the 8 lanes holding it
template <int B>
__device__ __forceinline__ void w4a16_stage4(f32x4 v, int t, int K, int nb, bool store,
                                             f32x4 *xs, float *sx) {
  asm volatile("" ::"v"(v));  // keep the load where it was issued
  const uint32_t h0 = bf16_pair(v.x, v.y), h1 = bf16_pair(v.z, v.w);
  const uint32_t l0 = bf16_pair(v.x - bf16_lo(h0), v.y - bf16_hi(h0));
  const uint32_t l1 = bf16_pair(v.z - bf16_lo(h1), v.w - bf16_hi(h1));
  // the sum of the values the products see (hi + lo), by dot products with 1
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  float s4 = __builtin_amdgcn_fdot2_f32_bf16(one, __builtin_bit_cast(bf16x2, h0), 0.0f, false);
  s4 = __builtin_amdgcn_fdot2_f32_bf16(one, __builtin_bit_cast(bf16x2, h1), s4, false);
  s4 = __builtin_amdgcn_fdot2_f32_bf16(one, __builtin_bit_cast(bf16x2, l0), s4, false);
  s4 = __builtin_amdgcn_fdot2_f32_bf16(one, __builtin_bit_cast(bf16x2, l1), s4, false);
  const float sum = group8_sum(s4);
  if (store) {  // uniform over each 8-lane group: the task count is a multiple of 8
    const int b = task_row<B>(t, K / 4), r = t - b * (K / 4), j = r >> 3, q = r & 7;
    xs[(b * 8 + q) * nb + j] = __builtin_bit_cast(f32x4, u32x4{h0, h1, l0, l1});
    if (q == 0) sx[b * nb + j] = -136.0f * sum;
  }
}

// Block j (the lane's) for RP weight rows and the B x rows: each code dword
// becomes two bf16 pairs once and serves every x row; x of all B rows for
// those positions is read from LDS once and serves the RP rows.  For each
// (row, x row) the sum starts at the staged -136 sum x and runs low nibbles
// then high nibbles, dwords ascending, per dword the hi parts of its four
// codes and then the lo parts; then acc += d_w * S.  (The x words are copied out of the vector before the
// bit cast: clang's __builtin_bit_cast of a vector element lvalue such as
// v.y reads element 0.)
template <int B, int RP>
__device__ __forceinline__ void w4a16_block(const u32x4 (&w)[RP], const float (&d)[RP],
                                            const f32x4 *xs, const float *sx, int nb, int j,
                                            float (&acc)[RP][B]) {
  constexpr int DG = B > 4 ? 2 : 4;  // code dwords per step (registers: x of B rows)
  float s1[RP][B];
#pragma unroll
  for (int r = 0; r < B; ++r) {
    const float c = sx[r * nb + j];
#pragma unroll
    for (int p = 0; p < RP; ++p) s1[p][r] = c;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {        // low nibbles: codes 0..15; high: 16..31
#pragma unroll
    for (int d0 = 0; d0 < 4; d0 += DG) {
      bf16x2 xq[B][DG][4];  // hi(x0 x1), hi(x2 x3), lo(x0 x1), lo(x2 x3)
#pragma unroll
      for (int r = 0; r < B; ++r)
#pragma unroll
        for (int dd = 0; dd < DG; ++dd) {
          const u32x4 v = __builtin_bit_cast(u32x4, xs[(r * 8 + 4 * h + d0 + dd) * nb + j]);
          const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) xq[r][dd][i] = __builtin_bit_cast(bf16x2, e[i]);
        }
#pragma unroll
      for (int p = 0; p < RP; ++p) {
        const uint32_t wd[4] = {w[p].x, w[p].y, w[p].z, w[p].w};
        bf16x2 a01[DG], a23[DG];
#pragma unroll
        for (int dd = 0; dd < DG; ++dd) {
          const uint32_t c = (wd[d0 + dd] >> (4 * h)) & 0x0F0F0F0Fu;
          // bytes {c0, 0x43, c1, 0x43}: bf16 128 + c0 and 128 + c1 (c < 128)
          a01[dd] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(0x43434343u, c, 0x04010400u));
          a23[dd] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(0x43434343u, c, 0x04030402u));
        }
#pragma unroll
        for (int r = 0; r < B; ++r)
#pragma unroll
          for (int dd = 0; dd < DG; ++dd) {
            float s = s1[p][r];
            s = __builtin_amdgcn_fdot2_f32_bf16(a01[dd], xq[r][dd][0], s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(a23[dd], xq[r][dd][1], s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(a01[dd], xq[r][dd][2], s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(a23[dd], xq[r][dd][3], s, false);
            s1[p][r] = s;
          }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < B; ++r)
#pragma unroll
    for (int p = 0; p < RP; ++p) acc[p][r] = fmaf(d[p], s1[p][r], acc[p][r]);
}

// K = 32 * G * T, or with RAG any K <= 32 * G * T (as in k_gemv_q4_0_t, a
// ragged row's last step loads its last block again and skips it), and
// B * K <= 16384 (x in at most 66 KiB of LDS): a workgroup owns one row
// group, every weight load of it issued up front.
template <int B, int G, int RP, int T, bool RAG, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_gemv_q4_0_f32(
    const uint8_t *__restrict__ qs, const uint16_t *__restrict__ dw, int N, int Kr,
    const float *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = RAG ? Kr : 32 * G * T, nb = K >> 5;  // RAG: the launcher checks K
  constexpr int NT = 64 * NW;  // threads per workgroup
  constexpr int RPP = 64 / G, ROWS_WAVE = RP * RPP, ROWS_WG = NW * ROWS_WAVE;
  const int TOT = B * K / 4;                              // float4 staging tasks
  f32x4 *xs = reinterpret_cast<f32x4 *>(smem);            // [B][8][nb]
  float *sx = reinterpret_cast<float *>(smem + (size_t)B * K * 4);  // [B][nb]
  const int lane = threadIdx.x & 63, sub = lane % G, grp = lane / G, wv = threadIdx.x >> 6;

  auto load_pass = [&](int base, auto &v) {
    constexpr int NP = sizeof(v) / sizeof(v[0]);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int t = min(base + (int)threadIdx.x + NT * m, TOT - 1);
      const int b = task_row<B>(t, K / 4), r = t - b * (K / 4);
      v[m] = load_f4(X + (int64_t)b * ldx + 4 * r);
    }
  };
  auto store_pass = [&](int base, const auto &v, int np) {
    constexpr int NP = sizeof(v) / sizeof(v[0]);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int t = base + threadIdx.x + NT * m;
      if (m < np) w4a16_stage4<B>(v[m], t, K, nb, t < TOT, xs, sx);
    }
  };

  // the first pass: kF32Pass tasks per thread, or for one ragged long row
  // all of x (8 G T / NT tasks) where the registers allow it
  constexpr int NALL = 8 * G * T / NT;
  constexpr int NP0 = (RAG && B == 1 && T <= 7 && NALL > kF32Pass) ? NALL : kF32Pass;
  const int P0 = min(NP0, (TOT + NT - 1) / NT);  // first-pass tasks per thread
  f32x4 xv[NP0];
  load_pass(0, xv);
  __builtin_amdgcn_sched_barrier(0);
  const int rbase = blockIdx.x * ROWS_WG + wv * ROWS_WAVE + grp;
  u32x4 w[T][RP];
  float d[T][RP];
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int64_t rowblk = (int64_t)min(rbase + p * RPP, N - 1) * nb;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t blk = rowblk + min(sub + G * t, nb - 1);
      w[t][p] = load_stream16(qs + blk * 16);
      d[t][p] = f16_bits_to_f32(load_stream2(dw + blk));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  store_pass(0, xv, P0);
  for (int base = NT * NP0; base < TOT; base += NT * kF32Pass) {
    f32x4 xr[kF32Pass];
    load_pass(base, xr);
    store_pass(base, xr, kF32Pass);
  }
  __syncthreads();

  float acc[RP][B];
#pragma unroll
  for (int p = 0; p < RP; ++p)
#pragma unroll
    for (int r = 0; r < B; ++r) acc[p][r] = 0.0f;
#pragma unroll
  for (int t = 0; t < T; ++t)  // the test is false only in the last step of a ragged row
    if (sub + G * t < nb) w4a16_block<B, RP>(w[t], d[t], xs, sx, nb, sub + G * t, acc);
  float (&flat)[RP * B] = *reinterpret_cast<float(*)[RP * B]>(&acc[0][0]);
  gsum_last_n<G>(flat);
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int row = rbase + p * RPP;
#pragma unroll
    for (int r = 0; r < B; ++r)
      if (sub == G - 1 && row < N) Y[(int64_t)r * ldy + row] = acc[p][r];
  }
}

// Any K % 32 == 0 with B * K <= MMV_Q4F32_MAX_XK: x of all B rows is staged
// once per workgroup (up to ~150 KiB of LDS, one workgroup per compute
// unit), and the workgroup walks row groups blockIdx.x, + gridDim.x, ...; a
// lane's blocks of a row group go in chunks of TC, the next chunk (or the
// next row group's first) in flight while the current one is multiplied.
// Blocks past the row are clamped in bounds and skipped.
template <int B, int G, int RP, int TC, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_gemv_q4_0_f32_g(
    const uint8_t *__restrict__ qs, const uint16_t *__restrict__ dw, int N, int K,
    const float *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int NT = 64 * NW;  // threads per workgroup
  constexpr int RPP = 64 / G, ROWS_WAVE = RP * RPP, ROWS_WG = NW * ROWS_WAVE;
  const int nb = K >> 5, tot = B * (K >> 2);
  const int nt = (nb + G - 1) / G;                          // blocks per lane and row
  const int nch = (nt + TC - 1) / TC;                       // chunks per row group
  const int ngroups = (N + ROWS_WG - 1) / ROWS_WG;
  f32x4 *xs = reinterpret_cast<f32x4 *>(smem);              // [B][8][nb]
  float *sx = reinterpret_cast<float *>(smem + (size_t)B * K * 4);  // [B][nb]
  const int lane = threadIdx.x & 63, sub = lane % G, grp = lane / G, wv = threadIdx.x >> 6;

  // the weights of chunk c of row group gi (blocks sub + G * (TC c + i))
  auto load_chunk = [&](int gi, int c, u32x4 (&w)[TC][RP], float (&d)[TC][RP]) {
    const int rbase = gi * ROWS_WG + wv * ROWS_WAVE + grp;
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      const int64_t rowblk = (int64_t)min(rbase + p * RPP, N - 1) * nb;
#pragma unroll
      for (int i = 0; i < TC; ++i) {
        const int64_t blk = rowblk + min(sub + G * (TC * c + i), nb - 1);
        w[i][p] = load_stream16(qs + blk * 16);
        d[i][p] = f16_bits_to_f32(load_stream2(dw + blk));
      }
    }
  };

  // x: a first pass of loads, then the first chunk of weights, then staging
  f32x4 xv[kF32Pass];
  auto load_pass = [&](int base) {
#pragma unroll
    for (int m = 0; m < kF32Pass; ++m) {
      const int t = min(base + (int)threadIdx.x + NT * m, tot - 1);
      const int b = task_row<B>(t, K / 4), r = t - b * (K / 4);
      xv[m] = load_f4(X + (int64_t)b * ldx + 4 * r);
    }
  };
  auto store_pass = [&](int base) {
#pragma unroll
    for (int m = 0; m < kF32Pass; ++m) {
      const int t = base + threadIdx.x + NT * m;
      w4a16_stage4<B>(xv[m], t, K, nb, t < tot, xs, sx);
    }
  };
  load_pass(0);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 wa[TC][RP], wb[TC][RP];
  float da[TC][RP], db[TC][RP];
  int gi = blockIdx.x;
  if (gi < ngroups) load_chunk(gi, 0, wa, da);  // uniform
  __builtin_amdgcn_sched_barrier(0);
  store_pass(0);
  for (int base = NT * kF32Pass; base < tot; base += NT * kF32Pass) {
    load_pass(base);
    store_pass(base);
  }
  __syncthreads();

  for (; gi < ngroups; gi += gridDim.x) {
    const int rbase = gi * ROWS_WG + wv * ROWS_WAVE + grp;
    float acc[RP][B];
#pragma unroll
    for (int p = 0; p < RP; ++p)
#pragma unroll
      for (int r = 0; r < B; ++r) acc[p][r] = 0.0f;
    for (int c = 0; c < nch; ++c) {
      // next: chunk c + 1 of this group, or chunk 0 of the next group
      const bool last = c + 1 == nch;
      const int gn = last ? gi + (int)gridDim.x : gi, cn = last ? 0 : c + 1;
      if (gn < ngroups) load_chunk(gn, cn, wb, db);  // uniform
#pragma unroll
      for (int i = 0; i < TC; ++i) {
        const int j = sub + G * (TC * c + i);
        if (j < nb) w4a16_block<B, RP>(wa[i], da[i], xs, sx, nb, j, acc);
      }
#pragma unroll
      for (int i = 0; i < TC; ++i)
#pragma unroll
        for (int p = 0; p < RP; ++p) {
          wa[i][p] = wb[i][p];
          da[i][p] = db[i][p];
        }
    }
    float (&flat)[RP * B] = *reinterpret_cast<float(*)[RP * B]>(&acc[0][0]);
    gsum_last_n<G>(flat);
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      const int row = rbase + p * RPP;
#pragma unroll
      for (int r = 0; r < B; ++r)
        if (sub == G - 1 && row < N) Y[(int64_t)r * ldy + row] = acc[p][r];
    }
  }
}

template <int B, int G, int RP>
static hipError_t launch_q4(const uint8_t *qs, const uint16_t *d, int N, int K,
                            const float *X, int64_t ldx, const uint8_t *Xq, float *Y,
                            int64_t ldy, hipStream_t s) {
  constexpr int rows_wg = 4 * RP * (64 / G);
  const int ngroups = (N + rows_wg - 1) / rows_wg;
  // workgroups per CU: each stages x once, so fewer when quantizing here
  const int knob = path_switch(MMV_PATH_Q4_WG_PER_CU);
  const int per_cu = knob ? knob : (X ? 2 : 4);
  const int blocks = min(ngroups, per_cu * cu_count());
  const size_t lds = xstage_bytes(B, K);
  hipLaunchKernelGGL((k_gemv_q4_0<B, G, RP>), dim3(blocks), dim3(256), lds, s, qs, d, N, K,
                     X, ldx, Xq, Y, ldy);
  return hipGetLastError();
}

template <int B, int G, int RP, int T, bool RAG = false, int NW = 4>
static hipError_t launch_q4_t(const uint8_t *qs, const uint16_t *d, int N, int K,
                              const float *X, int64_t ldx, const uint8_t *Xq, float *Y,
                              int64_t ldy, hipStream_t s) {
  constexpr int rows_wg = NW * RP * (64 / G);
  const int ngroups = (N + rows_wg - 1) / rows_wg;
  const size_t lds = xstage_bytes(B, K);
  if (X)
    hipLaunchKernelGGL((k_gemv_q4_0_t<B, G, RP, T, true, RAG, NW>), dim3(ngroups),
                       dim3(64 * NW), lds, s, qs, d, N, K, X, ldx, Xq, Y, ldy);
  else
    hipLaunchKernelGGL((k_gemv_q4_0_t<B, G, RP, T, false, RAG, NW>), dim3(ngroups),
                       dim3(64 * NW), lds, s, qs, d, N, K, X, ldx, Xq, Y, ldy);
  return hipGetLastError();
}

// B <= 4, a row of 64 < nb <= 512 blocks that is not a whole number of
// 64-block steps: the whole-row kernel with T = ceil(nb / 64) steps, the last
// one ragged, 4 rows per lane group (up to 32 weight blocks in flight per
// lane, 244 VGPRs at most, no spills; B * K <= MMV_Q4_MAX_XK keeps the staged
// x under 64 KiB).  Measured at 4096 x 11008 and 4096 x 14336, B = 1 / 2,
// against 2 rows per lane group (twice the workgroups, each quantizing x):
// 10.1 / 14.5 and 11.4 / 17.2 us against 10.9 / 16.4 and 12.8 / 20.1 us; the
// grid-stride kernel took 13.7 / 20.2 and 15.8 / 24.7 us (one block per lane
// in flight).  At B = 3 / 4 from a Q8_1 buffer, 4096 x 11008: 12.7 / 13.8
// against 19.2 / 20.8 us (from fp32 x: 20.7 / 24.9 against 28.7 / 33.8)
template <int B>
static hipError_t launch_q4_rag(const uint8_t *qs, const uint16_t *d, int N, int K,
                                const float *X, int64_t ldx, const uint8_t *Xq, float *Y,
                                int64_t ldy, hipStream_t s) {
  static_assert(B <= 4, "ragged whole-row launches are built for up to four rows");
  if constexpr (B == 1) {
    // one row: workgroups of 8 waves with 2 rows per lane group (the same 16
    // rows and grid), so each wave quantizes half as much of x and a SIMD
    // holds two waves: 4096 x 11008 9.8 -> 8.3 us, 4096 x 14336
    // 11.2 -> 9.5 us, 2560 x 9728 7.7 -> 6.6 us
    switch (((K >> 5) + 63) / 64) {
      case 2: return launch_q4_t<B, 64, 2, 2, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 3: return launch_q4_t<B, 64, 2, 3, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 4: return launch_q4_t<B, 64, 2, 4, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 5: return launch_q4_t<B, 64, 2, 5, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 6: return launch_q4_t<B, 64, 2, 6, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 7: return launch_q4_t<B, 64, 2, 7, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 8: return launch_q4_t<B, 64, 2, 8, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    }
  } else {  // also 8 waves of 2 rows per lane group (4096 x 11008, B = 2 / 3 / 4: from fp32 x
            // 14.5 / 20.7 / 24.9 -> 12.1 / 16.9 / 19.7 us, from a Q8_1 buffer 10.4 / 12.7 /
            // 13.7 -> 10.0 / 11.4 / 12.4 us)
    switch (((K >> 5) + 63) / 64) {
      case 2: return launch_q4_t<B, 64, 2, 2, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 3: return launch_q4_t<B, 64, 2, 3, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 4: return launch_q4_t<B, 64, 2, 4, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 5: return launch_q4_t<B, 64, 2, 5, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      case 6: return launch_q4_t<B, 64, 2, 6, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    }
    if constexpr (B <= 3) {  // B * K <= MMV_Q4_MAX_XK
      switch (((K >> 5) + 63) / 64) {
        case 7: return launch_q4_t<B, 64, 2, 7, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
        case 8: return launch_q4_t<B, 64, 2, 8, true, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      }
    }
  }
  return hipErrorInvalidValue;
}

// Rows per lane group of the 4-wave workgroups (2, 4, 6 or 8; the
// MMV_PATH_Q4_RP switch overrides): 4 by default.  (At B <= 4 the dispatch
// below prefers 8 waves of 2 rows per lane group where that measured
// faster.)
// Measured on the 4096 x 4096 and 11008 x 4096 shapes at B = 1, four rows
// per lane group (16 per workgroup) beat both two (twice the workgroups,
// each repeating the activation staging) and six or eight (fewer waves to
// overlap).  A lane holds at most 16 (B <= 2) or 8 weight blocks in flight.
template <int B, int G, int T>
static hipError_t launch_q4_rp(const uint8_t *qs, const uint16_t *d, int N, int K,
                               const float *X, int64_t ldx, const uint8_t *Xq, float *Y,
                               int64_t ldy, hipStream_t s) {
  constexpr int kMaxLoads = B <= 2 ? 16 : 8;
  constexpr int kMaxRp = cmin(8, (kMaxLoads / T) & ~1);
  // rows per lane group: 4, or 2 from B = 5 (more, smaller workgroups;
  // 4096^2 + 11008 x 4096 with a Q8_1 buffer, us per pair, RP 4 -> 2:
  // B = 5 18.7 -> 18.4, B = 6 20.2 -> 19.3, B = 8 22.7 -> 22.1; B = 4 level;
  // RP 8 at B = 8: 26.1)
  int rp = path_switch(MMV_PATH_Q4_RP);
  if (rp == 0) rp = B >= 5 ? 2 : cmin(4, kMaxRp);
  if constexpr (kMaxRp >= 8)
    if (rp > 6) return launch_q4_t<B, G, 8, T>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
  if constexpr (kMaxRp >= 6)
    if (rp > 4) return launch_q4_t<B, G, 6, T>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
  if constexpr (kMaxRp >= 4)
    if (rp > 2) return launch_q4_t<B, G, 4, T>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
  return launch_q4_t<B, G, 2, T>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
}

// shape of the matrix-core kernels (below)
constexpr int kMfW = 16;                  // waves per workgroup, each 1/16 of K
constexpr int kMfT = 64 * kMfW;           // threads per workgroup
constexpr int kMfCB = 8;                  // blocks per wave and tile, at most (K <= 4096)
constexpr int kMfLD = kMfCB / 4;          // 16-byte code loads and scales per lane and tile
constexpr int kMfXH = 1024 / kMfT;        // staging steps per thread (K / 4 <= 1024)
constexpr int kMfMaxXK = 32768;           // B * K: x planes in LDS
constexpr int kMfTileBytes = kMfCB * 272; // per wave: [block][row] 16 bytes, +16 per block

template <int B>
hipError_t launch_q4_mf(const uint8_t *qs, const uint16_t *d, int N, int K, const float *X,
                        int64_t ldx, const uint8_t *Xq, float *Y, int64_t ldy, hipStream_t s);

template <int B>
static hipError_t dispatch_q4(const uint8_t *qs, const uint16_t *d, int N, int K,
                              const float *X, int64_t ldx, const uint8_t *Xq, float *Y,
                              int64_t ldy, hipStream_t s) {
  const int nb = K / 32;
  constexpr int RP = B <= 2 ? 2 : 4;
  // K <= 4096: the matrix cores from B = 3 for fp32 x (quantized in every
  // workgroup: the dot4 kernels' repeated quantization is the bound there),
  // from B = 5 for a Q8_1 buffer (4096^2 + 11008 x 4096 per pair with the
  // quantization pass, dot4 / matrix cores: B = 4 16.5 / 16.9 us, B = 5
  // 18.0 / 17.7, B = 6 19.3 / 17.9)
  {
    const int sw = path_switch(MMV_PATH_Q4_MF);
    if (sw >= 0 && B >= (sw > 0 ? sw : (X ? 3 : 5)) && nb <= kMfW * kMfCB)
      return launch_q4_mf<B>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
  }
  // whole blocks per lane: every load of a row group in flight together
  if (path_switch(MMV_PATH_Q4_GENERIC) <= 0) {
    if (nb == 16) return launch_q4_rp<B, 16, 1>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    if (nb == 32) return launch_q4_rp<B, 32, 1>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    // two or four 64-block steps: workgroups of 8 waves, 2 rows per lane
    // group (the same 16 rows per workgroup; half of x's quantization or copy
    // per wave, two waves per SIMD) for one or two rows, and up to four rows
    // when the workgroup quantizes x itself, unless the rows-per-lane-group
    // switch asks for a 4-wave variant.  From a Q8_1 buffer at B = 3 / 4,
    // 4096 x 8192 measured 8.0 / 8.7 us with 4 waves against 8.4 / 9.1 with 8
    if constexpr (B <= 4)
      if ((B <= 2 || X) && path_switch(MMV_PATH_Q4_RP) == 0) {
        if (nb == 128) return launch_q4_t<B, 64, 2, 2, false, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
        if (nb == 256) return launch_q4_t<B, 64, 2, 4, false, 8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
      }
    if (nb == 64) return launch_q4_rp<B, 64, 1>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    if (nb == 128) return launch_q4_rp<B, 64, 2>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    if (nb == 256) return launch_q4_rp<B, 64, 4>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    if constexpr (B <= 4)
      if (nb > 64 && nb <= 512)
        return launch_q4_rag<B>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
  }
  if (nb <= 16) return launch_q4<B, 16, RP>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
  if (nb <= 32) return launch_q4<B, 32, RP>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
  return launch_q4<B, 64, RP>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
}

// ---- W4A16 on the matrix cores ------------------------------------------
// With B rows of x the fp32 kernels spend 32 FMAs per block, weight row and
// x row; v_mfma_f32_16x16x32_bf16 takes one Q4_0 block of 16 weight rows:
//  - A (16 rows x 32 k): lane l serves row l % 16 from the 4 code bytes
//    4 (l / 16) .. + 3 of the block, i.e. k = 4 (l / 16) + {0..3} (low
//    nibbles) and 16 + 4 (l / 16) + {0..3} (high nibbles), each code as the
//    bf16 value 128 + c (exact), one byte permute per two codes (0x43 is
//    the high byte of 128.0);
//  - B (32 k x 16 columns): x of the B rows as bf16 hi (columns 0..7) and
//    bf16 lo = bf16(x - hi) (columns 8..15; x - hi is exact in fp32),
//    stored in the same k order as A, so each lane reads its 8 values at
//    once; columns past B repeat row 0 and are never read back;
//  - per block and column: S = sum (128 + c) x_part - 136 sum x_part =
//    sum (c - 8) x_part (the accumulator starts at -136 sum x_part, the
//    block sums of x_part coming from the same instruction with A = 1),
//    then d_w S;
//  - y = the hi column plus the lo column, over the blocks.
// Rows agree with the fp32 kernels within rounding and bit for bit across
// every B this kernel takes (column b depends only on x row b).
// A workgroup of 16 waves stages x once, each wave keeps the x columns and
// block sums of its 1/16 of the blocks (at most 8: K <= 4096) in registers,
// and the workgroup walks 16-row tiles (persistent grid, one workgroup per
// CU: 4 waves per SIMD at <= 128 VGPRs). A wave's 16 rows x 8 blocks of
// codes arrive by row-contiguous 16-byte loads (8 lanes per row, 128 bytes)
// one tile ahead, and pass through the wave's own LDS tile into the A
// layout. (8 waves of 16 blocks measured the same for W4A16 and 10% slower
// for Q4_0 x Q8_1 from fp32 x, whose quantization then has half the threads.)
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// one tile of a wave: load i of lane l holds row (64 / kMfCB) i + l / kMfCB,
// block l % kMfCB of the wave's blocks (kMfCB lanes read a row's codes, one
// contiguous run); the scales of row l % 16 at blocks kMfLD (l / 16) + i.
// The two scales of a lane are adjacent: with D4 (an even number of blocks
// per row and per wave, and a 4-byte aligned scale plane) they come as one
// 4-byte load (a past-the-end pair is clamped to the row's last two blocks,
// which weigh 0 there), else as two 2-byte loads.  These loads touch each
// 64-byte line of scales from four lanes, so they keep the default cache
// policy: the non-temporal hint made the pair 1-1.5 us slower.  D4 is a
// template parameter: a run-time branch around the loads made the compiler
// wait for the next tile's code loads at its join.
struct MfChunk {
  u32x4 w[kMfLD];
  uint32_t dp;        // D4: the pair as loaded
  uint16_t d[kMfLD];  // else
  template <bool D4>
  __device__ __forceinline__ uint16_t scale(int i) const {
    if constexpr (D4) return (uint16_t)(dp >> (16 * i));
    else return d[i];
  }
};
static_assert(kMfLD == 2, "scale pairs");

template <bool D4>
__device__ __forceinline__ void mf_load(MfChunk &c, const uint8_t *__restrict__ qs,
                                        const uint16_t *__restrict__ dw, int N, int nb,
                                        int row0, int jb, int lane) {
  const int64_t jw = min(jb + lane % kMfCB, nb - 1);
#pragma unroll
  for (int i = 0; i < kMfLD; ++i) {
    const int64_t row = min(row0 + (64 / kMfCB) * i + lane / kMfCB, N - 1);
    c.w[i] = load_stream16(qs + (row * nb + jw) * 16);
  }
  const int64_t rowd = min(row0 + (lane & 15), N - 1);
  if constexpr (D4) {
    c.dp = *reinterpret_cast<const uint32_t *>(dw + rowd * nb + min(jb + 2 * (lane >> 4), nb - 2));
  } else {
#pragma unroll
    for (int i = 0; i < kMfLD; ++i)
      c.d[i] = dw[rowd * nb + min(jb + kMfLD * (lane >> 4) + i, nb - 1)];
  }
}

// The workgroup's tiles t, t + G, ... with two chunk buffers taken in turn:
// each tile but the last is computed with the next one's loads in flight,
// issued before the compute (unconditionally; the scheduling barrier keeps
// the compute below them).  Two named buffers instead of "cur = next": a
// register copy of a chunk waits for its loads, which left one tile's
// latency per tile.
template <bool D4, typename Tile>
__device__ __forceinline__ void mf_walk(MfChunk &a, MfChunk &b, int t, int G, int ntiles,
                                        const uint8_t *__restrict__ qs,
                                        const uint16_t *__restrict__ dw, int N, int nb, int jw0,
                                        int lane, Tile &tile) {
  // the first tile's loads, issued before x was staged, are in by now;
  // waiting for them here leaves the loop head no wait of its own (at the
  // merge of this state with the loop's, the compiler waited there for the
  // loads of the tile about to be computed)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  while (true) {  // every branch is uniform over the workgroup
    const int t2 = t + G;
    if (t2 >= ntiles) {
      tile(a, t);
      return;
    }
    mf_load<D4>(b, qs, dw, N, nb, 16 * t2, jw0, lane);
    __builtin_amdgcn_sched_barrier(0);
    tile(a, t);
    t = t2 + G;
    if (t >= ntiles) {
      tile(b, t2);
      return;
    }
    mf_load<D4>(a, qs, dw, N, nb, 16 * t, jw0, lane);
    __builtin_amdgcn_sched_barrier(0);
    tile(b, t2);
  }
}

// the scale pairs of mf_load as 4-byte loads: even blocks per row and per
// wave share (so every pair starts at an even block), aligned plane
inline bool mf_d4(const uint16_t *dw, int K) {
  const int nb = K >> 5, nbw = (nb + kMfW - 1) / kMfW;
  return ((nb | nbw) & 1) == 0 && (reinterpret_cast<uintptr_t>(dw) & 3) == 0;
}

template <int B, bool D4>
__global__ __launch_bounds__(kMfT) void k_gemv_q4_0_f32_mf(
    const uint8_t *__restrict__ qs, const uint16_t *__restrict__ dw, int N, int K,
    const float *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];    // x planes, then the waves' code tiles
  __shared__ __align__(16) float s_d[kMfW][kMfCB][16];  // [wave][block][row] scales
  __shared__ float s_part[2][kMfW][16][9];              // [parity][wave][row][b] tile sums
  const int nb = K >> 5, KP = K + 8;
  uint16_t *xpl = reinterpret_cast<uint16_t *>(smem);  // [2B][KP] bf16
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int ntiles = (N + 15) >> 4;
  const int nbw = (nb + kMfW - 1) / kMfW;  // blocks per wave and tile (<= kMfCB)
  const int jw0 = min(nb, wv * nbw), jw1 = min(nb, jw0 + nbw);
  int t = blockIdx.x;
  const int G = gridDim.x;

  // x (kMfXH float4 per row and thread: K <= 4096), then the first tile's
  // codes, in this order so that staging x waits for x only; x -> hi / lo
  // planes in the k order of the A operand
  const int k4 = K >> 2;
  f32x4 v[kMfXH][B];
#pragma unroll
  for (int h = 0; h < kMfXH; ++h) {
    const int kk = min(kMfT * h + tid, k4 - 1);
#pragma unroll
    for (int b = 0; b < B; ++b) v[h][b] = load_f4(X + (int64_t)b * ldx + 4 * kk);
  }
  __builtin_amdgcn_sched_barrier(0);
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  u32x4 xreg[kMfCB];
  f32x4 creg[kMfCB];  // -136 sum x_part in all four entries: the accumulator S starts from
  MfChunk cur;
  mf_load<D4>(cur, qs, dw, N, nb, 16 * t, jw0, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < kMfXH; ++h) {
    // (no test: past K / 4 a thread repeats the last float4, same value to
    // the same place, so that no load moves into a branch)
    const int kk = min(kMfT * h + tid, k4 - 1);
    {
      const int k = 4 * kk, q = k & 31;
      const int pos = (k - q) + 2 * (q & 12) + ((q >> 2) & 4);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const f32x4 x4 = v[h][b];
        const uint32_t h0 =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x4.x, x4.y}, bf16x2));
        const uint32_t h1 =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x4.z, x4.w}, bf16x2));
        const uint32_t l0 = __builtin_bit_cast(
            uint32_t,
            __builtin_convertvector(f32x2{x4.x - bf16_lo(h0), x4.y - bf16_hi(h0)}, bf16x2));
        const uint32_t l1 = __builtin_bit_cast(
            uint32_t,
            __builtin_convertvector(f32x2{x4.z - bf16_lo(h1), x4.w - bf16_hi(h1)}, bf16x2));
        *reinterpret_cast<u32x2 *>(xpl + (size_t)b * KP + pos) = u32x2{h0, h1};
        *reinterpret_cast<u32x2 *>(xpl + (size_t)(B + b) * KP + pos) = u32x2{l0, l1};
      }
    }
  }
  __syncthreads();

  // this lane's B column (plane row (col / 8) B + col % 8, row 0 past B)
  // at the wave's blocks, and 136 * its block sums (A = 1)
  {
    const int bc = (col & 7) < B ? (col & 7) : 0;
    const uint16_t *xrow = xpl + (size_t)((col >> 3) * B + bc) * KP + 8 * kg;
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
    for (int u = 0; u < kMfCB; ++u) {
      xreg[u] = *reinterpret_cast<const u32x4 *>(xrow + 32 * min(jw0 + u, nb - 1));
      const f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8v, ones), __builtin_bit_cast(bf16x8v, xreg[u]), zero, 0, 0,
          0);
      const float c = -136.0f * s.x;
      creg[u] = f32x4{c, c, c, c};
    }
  }
  __syncthreads();  // the x planes are dead: the code tiles take their place

  uint8_t *wt = smem + wv * kMfTileBytes;
  float *sdw = &s_d[wv][0][0];
  int par = 0;
  // one tile: codes to the A layout ([block][row] 16 bytes), scales as fp32
  // [block][row] (blocks past the wave's share weigh 0), the 16 blocks, then
  // the lo column onto the hi column (lanes col + 8 -> col) and the 8 waves'
  // shares; the next tile writes the other parity of s_part, the one after
  // that comes after the next barrier, when these reads are done
  auto tile = [&](const MfChunk &c, int tt) {
#pragma unroll
    for (int i = 0; i < kMfLD; ++i)
      *reinterpret_cast<u32x4 *>(wt + (lane % kMfCB) * 272 +
                                 ((64 / kMfCB) * i + lane / kMfCB) * 16) = c.w[i];
#pragma unroll
    for (int i = 0; i < kMfLD; ++i)
      sdw[(kMfLD * kg + i) * 16 + col] =
          jw0 + kMfLD * kg + i < jw1 ? f16_bits_to_f32(c.template scale<D4>(i)) : 0.0f;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's tile stores
    __builtin_amdgcn_wave_barrier();
    f32x4 acc = zero;
#pragma unroll
    for (int u = 0; u < kMfCB; ++u) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(wt + u * 272 + col * 16 + 4 * kg);
      const uint32_t mlo = w & 0x0F0F0F0Fu, mhi = (w >> 4) & 0x0F0F0F0Fu;
      u32x4 av;
      av.x = __builtin_amdgcn_perm(0x43434343u, mlo, 0x04010400u);
      av.y = __builtin_amdgcn_perm(0x43434343u, mlo, 0x04030402u);
      av.z = __builtin_amdgcn_perm(0x43434343u, mhi, 0x04010400u);
      av.w = __builtin_amdgcn_perm(0x43434343u, mhi, 0x04030402u);
      // S - 136 sum x_part (the accumulator starts from the correction)
      const f32x4 s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8v, av), __builtin_bit_cast(bf16x8v, xreg[u]), creg[u], 0, 0,
          0);
      // scales of rows 4 kg .. 4 kg + 3 at this block
      const f32x4 sd = *reinterpret_cast<const f32x4 *>(sdw + u * 16 + 4 * kg);
      acc.x = fmaf(sd.x, s4.x, acc.x);
      acc.y = fmaf(sd.y, s4.y, acc.y);
      acc.z = fmaf(sd.z, s4.z, acc.z);
      acc.w = fmaf(sd.w, s4.w, acc.w);
    }
    __builtin_amdgcn_wave_barrier();  // the tile and s_d are rewritten next time
    acc.x += dpp_f32<0x128>(acc.x);   // row_ror:8
    acc.y += dpp_f32<0x128>(acc.y);
    acc.z += dpp_f32<0x128>(acc.z);
    acc.w += dpp_f32<0x128>(acc.w);
    if (col < B) {
      s_part[par][wv][4 * kg + 0][col] = acc.x;
      s_part[par][wv][4 * kg + 1][col] = acc.y;
      s_part[par][wv][4 * kg + 2][col] = acc.z;
      s_part[par][wv][4 * kg + 3][col] = acc.w;
    }
    __syncthreads();
    if (tid < 16 * B) {
      const int b = tid >> 4, row = tid & 15;
      float v = 0.0f;
#pragma unroll
      for (int w8 = 0; w8 < kMfW; ++w8) v += s_part[par][w8][row][b];
      const int n = 16 * tt + row;
      if (n < N) Y[(int64_t)b * ldy + n] = v;
    }
    par ^= 1;
  };
  // every tile but the last with the next one's loads in flight (issued
  // before the compute, unconditionally, so that only this tile's loads
  // have to land); the last one without.  (mf_walk's two buffers, as the
  // int8 kernel walks its tiles, measured 0.3 us slower per pair here at
  // B = 2 / 3: at 128 VGPRs they spill.)
  while (true) {
    const int t2 = t + G;
    if (t2 >= ntiles) break;  // uniform over the workgroup
    MfChunk nxt;
    mf_load<D4>(nxt, qs, dw, N, nb, 16 * t2, jw0, lane);
    tile(cur, t);
    t = t2;
    cur = nxt;
  }
  tile(cur, t);
}

// ---- Q4_0 x Q8_1 on the matrix cores -------------------------------------
// The same tiling as W4A16 on the matrix cores, with v_mfma_i32_16x16x64_i8
// on two blocks at once (int8 needs no hi / lo columns, so the 16 columns
// hold 8 x rows twice: block j in columns 0..7, block j + 1 in 8..15):
//  - A (16 rows x 64 k): lanes 0..31 serve block j, 32..63 block j + 1;
//    lane l takes the 8 code bytes 8 ((l / 16) % 2) .. + 7 of its block,
//    masked into 8 low-nibble and 8 high-nibble codes (unsigned int8 0..15);
//  - B (64 k x 16 columns): column c < 8 holds the Q8_1 codes of x row c at
//    block j in lanes 0..31 and zeros in 32..63, column c + 8 the same row
//    at block j + 1 in lanes 32..63 and zeros in 0..31; the x codes sit in
//    LDS in the k order of A, so a lane reads its 16 at once;
//  - per block and x row: S = sum code * q (exact int32), I = S - 8 sum q
//    (sum q from the same instruction with A = 1), then y += (d_w d_x) I in
//    fp32 -- I is the block's exact integer dot of the W4A8 product; column
//    c + 8 folds onto column c at the end.
// x comes as fp32 (quantized to Q8_1 in every workgroup by the one device
// routine, so the codes equal the standalone quantizer's) or as a Q8_1
// buffer. Rows are bit-identical across every B this kernel takes.
template <int B, bool FROM_X, bool D4>
__global__ __launch_bounds__(kMfT) void k_gemv_q4_0_mf(
    const uint8_t *__restrict__ qs, const uint16_t *__restrict__ dw, int N, int K,
    const float *__restrict__ X, int64_t ldx, const uint8_t *__restrict__ Xq,
    float *__restrict__ Y, int64_t ldy) {
  // x codes and scales, then the code tiles (typed views of one dynamic
  // LDS block, indexed in 32 bits)
  extern __shared__ __align__(16) uint8_t smem[];
  extern __shared__ __align__(16) uint32_t smem_u[];
  extern __shared__ __align__(16) float smem_f[];
  __shared__ __align__(16) float s_d[kMfW][kMfCB][16];  // [wave][block][row] weight scales
  __shared__ float s_part[2][kMfW][16][9];              // [parity][wave][row][b] tile sums
  const int nb = K >> 5, KP = K + 16;
  // [B][KP] int8 codes at smem (bytes K .. K + 15 of a row unused), then
  // [B][nb] fp32 x scales and one spare word, from word dx0
  const unsigned dx0 = B * KP / 4;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int ntiles = (N + 15) >> 4;
  const int nbw = (nb + kMfW - 1) / kMfW;  // blocks per wave and tile (<= kMfCB)
  const int jw0 = min(nb, wv * nbw), jw1 = min(nb, jw0 + nbw);
  int t = blockIdx.x;
  const int G = gridDim.x;

  // x (kMfXH groups of 4 values per row and thread: K <= 4096), then
  // the first tile's codes, in this order so that staging x waits for x
  // only; the x codes go to LDS in the k order of the A operand
  const int k4 = K >> 2;
  f32x4 v[FROM_X ? kMfXH : 1][FROM_X ? B : 1];
  uint32_t c[FROM_X ? 1 : kMfXH][FROM_X ? 1 : B];
  uint16_t dq[FROM_X ? 1 : kMfXH];  // x scales of a Q8_1 buffer: B * nb <= 1024
#pragma unroll
  for (int h = 0; h < kMfXH; ++h) {
    const int kk = min(kMfT * h + tid, k4 - 1);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if constexpr (FROM_X)
        v[h][b] = load_f4(X + (int64_t)b * ldx + 4 * kk);
      else
        c[h][b] = *reinterpret_cast<const uint32_t *>(Xq + (size_t)b * K + 4 * kk);
    }
    if constexpr (!FROM_X)
      dq[h] = reinterpret_cast<const uint16_t *>(Xq + (size_t)B * K)[2 * min(kMfT * h + tid, B * nb - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);
  MfChunk cur;
  mf_load<D4>(cur, qs, dw, N, nb, 16 * t, jw0, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < kMfXH; ++h) {
    // past K / 4 a thread works on the last group of 4 values and stores
    // into unused words (no branch, so that no load moves into one); Q8_1
    // takes whole 8-lane groups (32 values), which K % 32 == 0 keeps either
    // wholly inside or wholly past the row
    // (row offsets as running sums: a multiply-add here becomes a 64-bit
    // one whose unused half reads a register with a load in flight)
    const int kr = kMfT * h + tid, kk = min(kr, k4 - 1);
    const bool in = kr < k4, lead = in && (kk & 7) == 0;
    const unsigned k = 4 * kk, q = k & 31;
    unsigned cw = (in ? (k - q) + 16 * ((q >> 3) & 1) + (q & 7) + 8 * (q >> 4) : (unsigned)K) >> 2;
    unsigned di = dx0 + (kk >> 3);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      uint32_t codes;
      if constexpr (FROM_X) {
        const Q8Block qb = q8_1_quantize8(v[h][b]);
        codes = qb.codes;
        smem_f[lead ? di : dx0 + B * nb] = f16_bits_to_f32(qb.d16);
      } else {
        codes = c[h][b];
      }
      smem_u[cw] = codes;
      cw += KP >> 2;
      di += nb;
    }
    if constexpr (!FROM_X) {
      const int i = kMfT * h + tid;
      smem_f[i < B * nb ? dx0 + i : dx0 + B * nb] = f16_bits_to_f32(dq[h]);
    }
  }
  __syncthreads();

  // this lane's B operand per block pair (x row col % 8, row 0 past B; its
  // 16 codes, or zeros where its column takes the other block of the pair),
  // and its column's scale and 8 * code sum (A = 1)
  typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
  const i32x4v izero = {0, 0, 0, 0};
  constexpr int NP = kMfCB / 2;  // block pairs per wave and tile
  i32x4v xq[NP];
  float dx[NP];
  i32x4v nq8[NP];  // -8 sum q in all four entries: the accumulator the block dot starts from
  {
    const int bc = (col & 7) < B ? (col & 7) : 0;
    const bool mine = (col >= 8) == (kg >= 2);
    const int xrow = (bc * KP + 16 * (kg & 1)) >> 2;
    const i32x4v ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int jb = min(jw0 + 2 * p + (kg >> 1), nb - 1);   // this lane's B rows
      const int jc = min(jw0 + 2 * p + (col >> 3), nb - 1);  // this lane's column
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&smem_u[xrow + 8 * jb]);
      xq[p] = mine ? __builtin_bit_cast(i32x4v, v) : izero;
      dx[p] = smem_f[dx0 + bc * nb + jc];
      const i32x4v s = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, xq[p], izero, 0, 0, 0);
      nq8[p] = i32x4v{-8 * s.x, -8 * s.x, -8 * s.x, -8 * s.x};
    }
  }
  __syncthreads();  // x is in registers: the code tiles take its place

  const int wt = wv * kMfTileBytes / 4;  // this wave's code tile, in words
  float *sdw = &s_d[wv][0][0];
  int par = 0;
  // one tile, as in the W4A16 kernel (s_part parities alternate)
  auto tile = [&](const MfChunk &ch, int tt) {
#pragma unroll
    for (int i = 0; i < kMfLD; ++i)
      *reinterpret_cast<u32x4 *>(
          &smem_u[wt + (lane % kMfCB) * 68 + ((64 / kMfCB) * i + lane / kMfCB) * 4]) = ch.w[i];
#pragma unroll
    for (int i = 0; i < kMfLD; ++i)
      sdw[(kMfLD * kg + i) * 16 + col] =
          jw0 + kMfLD * kg + i < jw1 ? f16_bits_to_f32(ch.template scale<D4>(i)) : 0.0f;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's tile stores
    __builtin_amdgcn_wave_barrier();
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      // A: row col, block 2p + kg / 2, code bytes 8 (kg % 2) .. + 7
      const u32x2 w = *reinterpret_cast<const u32x2 *>(
          &smem_u[wt + (2 * p + (kg >> 1)) * 68 + col * 4 + 2 * (kg & 1)]);
      i32x4v a;
      a.x = (int)(w.x & 0x0F0F0F0Fu);
      a.y = (int)(w.y & 0x0F0F0F0Fu);
      a.z = (int)((w.x >> 4) & 0x0F0F0F0Fu);
      a.w = (int)((w.y >> 4) & 0x0F0F0F0Fu);
      // I = sum code * q - 8 sum q, exact
      const i32x4v i4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xq[p], nq8[p], 0, 0, 0);
      // this lane's outputs: rows 4 kg .. + 3 of column col, block 2p + col / 8
      const f32x4 sd = *reinterpret_cast<const f32x4 *>(sdw + (2 * p + (col >> 3)) * 16 + 4 * kg);
      const float d = dx[p];
      acc.x = fmaf(sd.x * d, (float)i4.x, acc.x);
      acc.y = fmaf(sd.y * d, (float)i4.y, acc.y);
      acc.z = fmaf(sd.z * d, (float)i4.z, acc.z);
      acc.w = fmaf(sd.w * d, (float)i4.w, acc.w);
    }
    __builtin_amdgcn_wave_barrier();  // the tile and s_d are rewritten next time
    acc.x += dpp_f32<0x128>(acc.x);   // row_ror:8: the odd blocks (columns 8..15) onto
    acc.y += dpp_f32<0x128>(acc.y);   // the even ones (columns 0..7)
    acc.z += dpp_f32<0x128>(acc.z);
    acc.w += dpp_f32<0x128>(acc.w);
    if (col < B) {
      s_part[par][wv][4 * kg + 0][col] = acc.x;
      s_part[par][wv][4 * kg + 1][col] = acc.y;
      s_part[par][wv][4 * kg + 2][col] = acc.z;
      s_part[par][wv][4 * kg + 3][col] = acc.w;
    }
    __syncthreads();
    if (tid < 16 * B) {
      const int b = tid >> 4, row = tid & 15;
      float v8 = 0.0f;
#pragma unroll
      for (int w8 = 0; w8 < kMfW; ++w8) v8 += s_part[par][w8][row][b];
      const int n = 16 * tt + row;
      if (n < N) Y[(int64_t)b * ldy + n] = v8;
    }
    par ^= 1;
  };
  MfChunk nxt;
  mf_walk<D4>(cur, nxt, t, G, ntiles, qs, dw, N, nb, jw0, lane, tile);
}

// a persistent grid, one 16-wave workgroup per CU
template <int B>
hipError_t launch_q4_mf(const uint8_t *qs, const uint16_t *d, int N, int K, const float *X,
                        int64_t ldx, const uint8_t *Xq, float *Y, int64_t ldy, hipStream_t s) {
  const size_t xb = (size_t)B * (K + 16) + (size_t)4 * B * (K / 32) + 4;
  const size_t tiles = (size_t)kMfW * kMfTileBytes;
  const size_t lds = xb > tiles ? xb : tiles;  // at most 41 KiB (B = 8, K = 4096)
  const int grid = min((N + 15) / 16, cu_count());
  const bool d4 = mf_d4(d, K);
  if (X && d4)
    hipLaunchKernelGGL((k_gemv_q4_0_mf<B, true, true>), dim3(grid), dim3(kMfT), lds, s, qs, d, N,
                       K, X, ldx, Xq, Y, ldy);
  else if (X)
    hipLaunchKernelGGL((k_gemv_q4_0_mf<B, true, false>), dim3(grid), dim3(kMfT), lds, s, qs, d,
                       N, K, X, ldx, Xq, Y, ldy);
  else if (d4)
    hipLaunchKernelGGL((k_gemv_q4_0_mf<B, false, true>), dim3(grid), dim3(kMfT), lds, s, qs, d,
                       N, K, X, ldx, Xq, Y, ldy);
  else
    hipLaunchKernelGGL((k_gemv_q4_0_mf<B, false, false>), dim3(grid), dim3(kMfT), lds, s, qs, d,
                       N, K, X, ldx, Xq, Y, ldy);
  return hipGetLastError();
}

namespace {

template <int B, int G, int T, bool RAG = false, int NW = 4>
hipError_t launch_q4_f32(const uint8_t *qs, const uint16_t *d, int N, int K, const float *X,
                         int64_t ldx, float *Y, int64_t ldy, hipStream_t s) {
  // rows per lane group: 2 for the 8192-long rows, 4 otherwise (ragged rows:
  // 4096 x 11008 at B = 1 11.0 against 11.6 us with 2); 8-wave workgroups
  // keep the workgroup's rows with half as many per lane group
  constexpr int RP = ((T >= 4 && !RAG) ? 2 : 4) * 4 / NW;
  constexpr int rows_wg = NW * RP * (64 / G);
  const size_t lds = (size_t)B * K * 4 + (size_t)B * (K / 32) * 4;
  if (lds > 65536) {  // above the default dynamic-LDS limit: raise it once per kernel
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_gemv_q4_0_f32<B, G, RP, T, RAG, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 32 * G * T * B * 4 + G * T * B * 4);
    if (raised != hipSuccess) return raised;
  }
  hipLaunchKernelGGL((k_gemv_q4_0_f32<B, G, RP, T, RAG, NW>), dim3((N + rows_wg - 1) / rows_wg),
                     dim3(64 * NW), lds, s, qs, d, N, K, X, ldx, Y, ldy);
  return hipGetLastError();
}

// B <= 3 and 64 < nb <= 512 blocks: the whole-row kernel with T =
// ceil(nb / 64) steps, the last one ragged where nb is not a multiple of 64
// (B * K <= MMV_Q4F32_MAX_XK: T <= 8 for one or two rows, T <= 6 for three;
// above 64 KiB of staged x the launcher raises the workgroup's LDS limit)
template <int B>
hipError_t launch_q4_f32_rag(const uint8_t *qs, const uint16_t *d, int N, int K, const float *X,
                             int64_t ldx, float *Y, int64_t ldy, hipStream_t s) {
  static_assert(B <= 3, "ragged whole-row launches are built for up to three rows");
  if constexpr (B == 1) {
    // one row of three or more steps: 8-wave workgroups with 2 rows per lane
    // group (4096 x 11008 10.95 -> 10.35 us, 4096 x 14336 12.4 -> 11.8 us;
    // two steps measured slower: 9728 x 2560 7.3 -> 7.7 us)
    switch (((K >> 5) + 63) / 64) {
      case 2: return launch_q4_f32<B, 64, 2, true>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 3: return launch_q4_f32<B, 64, 3, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 4: return launch_q4_f32<B, 64, 4, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 5: return launch_q4_f32<B, 64, 5, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 6: return launch_q4_f32<B, 64, 6, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 7: return launch_q4_f32<B, 64, 7, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 8: return launch_q4_f32<B, 64, 8, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
    }
  } else {  // two or three rows: 8-wave workgroups at every step count (4096 x 11008
            // B = 2 / 3 14.9 / 21.1 -> 14.2 / 19.5 us, 2560 x 9728 B = 3 16.9 -> 14.9 us,
            // 4096 x 6144 B = 2 8.95 -> 7.94 us)
    switch (((K >> 5) + 63) / 64) {
      case 2: return launch_q4_f32<B, 64, 2, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 3: return launch_q4_f32<B, 64, 3, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 4: return launch_q4_f32<B, 64, 4, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 5: return launch_q4_f32<B, 64, 5, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 6: return launch_q4_f32<B, 64, 6, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
    }
    if constexpr (B == 2) {  // B * K <= MMV_Q4F32_MAX_XK
      switch (((K >> 5) + 63) / 64) {
        case 7: return launch_q4_f32<B, 64, 7, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
        case 8: return launch_q4_f32<B, 64, 8, true, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
      }
    }
  }
  return hipErrorInvalidValue;
}

// W4A16 on the matrix cores: a persistent grid, one 16-wave workgroup per CU
template <int B, bool D4>
hipError_t launch_q4_f32_mf_d(const uint8_t *qs, const uint16_t *d, int N, int K,
                              const float *X, int64_t ldx, float *Y, int64_t ldy,
                              hipStream_t s) {
  constexpr size_t kMaxLds = (size_t)4 * kMfMaxXK + (size_t)4 * B * 8;
  const size_t xb = (size_t)4 * B * (K + 8), tiles = (size_t)kMfW * kMfTileBytes;
  const size_t lds = xb > tiles ? xb : tiles;
  if (lds > 65536) {  // above the default dynamic-LDS limit: raise it once per kernel
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_gemv_q4_0_f32_mf<B, D4>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (raised != hipSuccess) return raised;
  }
  const int grid = min((N + 15) / 16, cu_count());
  hipLaunchKernelGGL((k_gemv_q4_0_f32_mf<B, D4>), dim3(grid), dim3(kMfT), lds, s, qs, d, N, K,
                     X, ldx, Y, ldy);
  return hipGetLastError();
}

template <int B>
hipError_t launch_q4_f32_mf(const uint8_t *qs, const uint16_t *d, int N, int K, const float *X,
                            int64_t ldx, float *Y, int64_t ldy, hipStream_t s) {
  return mf_d4(d, K) ? launch_q4_f32_mf_d<B, true>(qs, d, N, K, X, ldx, Y, ldy, s)
                     : launch_q4_f32_mf_d<B, false>(qs, d, N, K, X, ldx, Y, ldy, s);
}

// the general kernel with NW waves per workgroup
template <int B, int G, int TC, int NW>
hipError_t launch_q4_f32_gw(const uint8_t *qs, const uint16_t *d, int N, int K, const float *X,
                            int64_t ldx, float *Y, int64_t ldy, hipStream_t s) {
  constexpr int RP = 2;
  constexpr int rows_wg = NW * RP * (64 / G);
  constexpr size_t kMaxLds = (size_t)MMV_Q4F32_MAX_XK * 4 + (size_t)MMV_Q4F32_MAX_XK / 32 * 4;
  const size_t lds = (size_t)B * K * 4 + (size_t)B * (K / 32) * 4;
  if (lds > 65536) {  // above the default dynamic-LDS limit: raise it once per kernel
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_gemv_q4_0_f32_g<B, G, RP, TC, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (raised != hipSuccess) return raised;
  }
  const int ngroups = (N + rows_wg - 1) / rows_wg;
  const int per_cu = lds > 81920 ? 1 : 2;
  const int grid = min(ngroups, per_cu * cu_count());
  hipLaunchKernelGGL((k_gemv_q4_0_f32_g<B, G, RP, TC, NW>), dim3(grid), dim3(64 * NW), lds, s,
                     qs, d, N, K, X, ldx, Y, ldy);
  return hipGetLastError();
}

// the general kernel: x of all rows in LDS (up to the B * K limit), one
// workgroup per compute unit when that takes more than 80 KiB, and then 8
// waves of 2 rows per lane group (16-row groups): 8192 x 28672 at B = 1
// 41.1 -> 33.7 us, 4096 x 18432 at B = 2 24.2 -> 20.4 us, 11008 x 8192 at
// B = 3 31.4 -> 25.6 us.  With two workgroups per CU the 16-row groups split
// unevenly (14336 x 6144, B = 3: 25.9 -> 31.4 us), so 4 waves stay there, and
// from B = 4 the 8-wave instances spill registers.
template <int B, int G, int TC>
hipError_t launch_q4_f32_g(const uint8_t *qs, const uint16_t *d, int N, int K, const float *X,
                           int64_t ldx, float *Y, int64_t ldy, hipStream_t s) {
  const size_t lds = (size_t)B * K * 4 + (size_t)B * (K / 32) * 4;
  if constexpr (G == 64 && B <= 3)
    if (lds > 81920) return launch_q4_f32_gw<B, G, TC, 8>(qs, d, N, K, X, ldx, Y, ldy, s);
  return launch_q4_f32_gw<B, G, TC, 4>(qs, d, N, K, X, ldx, Y, ldy, s);
}

template <int B>
hipError_t dispatch_q4_f32(const uint8_t *qs, const uint16_t *d, int N, int K, const float *X,
                           int64_t ldx, float *Y, int64_t ldy, hipStream_t s) {
  const int nb = K / 32;
  // two or more rows and K <= 4096: the matrix cores
  {
    const int sw = path_switch(MMV_PATH_Q4F32_MF);
    if (sw >= 0 && B >= (sw > 0 ? sw : 2) && nb <= kMfW * kMfCB && (int64_t)B * K <= kMfMaxXK)
      return launch_q4_f32_mf<B>(qs, d, N, K, X, ldx, Y, ldy, s);
  }
  // whole rows per lane, one row group per workgroup: x of B rows in at
  // most 66 KiB of LDS
  if ((int64_t)B * K <= 16384) {
    switch (nb) {
      case 16: return launch_q4_f32<B, 16, 1>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 32: return launch_q4_f32<B, 32, 1>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 64: return launch_q4_f32<B, 64, 1>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 128:  // one row: 8-wave workgroups, as for the W4A8 kernel
        return launch_q4_f32<B, 64, 2, false, B == 1 ? 8 : 4>(qs, d, N, K, X, ldx, Y, ldy, s);
      case 256: return launch_q4_f32<B, 64, 4>(qs, d, N, K, X, ldx, Y, ldy, s);
      default: break;
    }
  }
  // ragged rows (and whole ones past 16384 = B * K): the whole-row kernel
  // with a ragged last step, above B * K = 16384 only when its workgroups of
  // 16 rows fit the CUs in one round (x of all B rows, up to 152 KiB, is
  // staged by every workgroup; at 11008 x 8192 and 14336 x 6144, B = 3, two
  // or more rounds took 39.1 and 33.2 us against 31.2 and 25.5 us on the
  // general kernel, which stages x once per CU)
  if constexpr (B <= 3)
    if (nb > 64 && nb <= 512 && (int64_t)B * K <= MMV_Q4F32_MAX_XK) {
      const int64_t lds = (int64_t)B * K * 4 + (int64_t)B * nb * 4;
      const int per_cu = (int)(163840 / lds);
      if ((int64_t)B * K <= 16384 || (N + 15) / 16 <= per_cu * cu_count())
        return launch_q4_f32_rag<B>(qs, d, N, K, X, ldx, Y, ldy, s);
    }
  // any other K, or more rows: the general kernel with the same lanes per
  // row (hence the same per-row order and bits)
  constexpr int TC = B > 4 ? 2 : 4;
  if (nb <= 16) return launch_q4_f32_g<B, 16, TC>(qs, d, N, K, X, ldx, Y, ldy, s);
  if (nb <= 32) return launch_q4_f32_g<B, 32, TC>(qs, d, N, K, X, ldx, Y, ldy, s);
  return launch_q4_f32_g<B, 64, TC>(qs, d, N, K, X, ldx, Y, ldy, s);
}

}  // namespace

hipError_t run_gemv_q4_0_f32(const uint8_t *qs, const uint16_t *d, int N, int K,
                             const float *X, int64_t ldx, int B, float *Y, int64_t ldy,
                             hipStream_t s) {
  switch (B) {
    case 1: return dispatch_q4_f32<1>(qs, d, N, K, X, ldx, Y, ldy, s);
    case 2: return dispatch_q4_f32<2>(qs, d, N, K, X, ldx, Y, ldy, s);
    case 3: return dispatch_q4_f32<3>(qs, d, N, K, X, ldx, Y, ldy, s);
    case 4: return dispatch_q4_f32<4>(qs, d, N, K, X, ldx, Y, ldy, s);
    case 5: return dispatch_q4_f32<5>(qs, d, N, K, X, ldx, Y, ldy, s);
    case 6: return dispatch_q4_f32<6>(qs, d, N, K, X, ldx, Y, ldy, s);
    case 7: return dispatch_q4_f32<7>(qs, d, N, K, X, ldx, Y, ldy, s);
    case 8: return dispatch_q4_f32<8>(qs, d, N, K, X, ldx, Y, ldy, s);
  }
  return hipErrorInvalidValue;
}

hipError_t run_gemv_q4_0(const uint8_t *qs, const uint16_t *d, int N, int K,
                         const float *X, int64_t ldx, const uint8_t *Xq, int B,
                         float *Y, int64_t ldy, hipStream_t s) {
  if (X && Xq) {  // quantize once into the caller's buffer, then read it
    const hipError_t e = run_quantize_q8_1(X, K, ldx, B, const_cast<uint8_t *>(Xq), s);
    if (e != hipSuccess) return e;
    X = nullptr;
  }
  switch (B) {
    case 1: return dispatch_q4<1>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    case 2: return dispatch_q4<2>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    case 3: return dispatch_q4<3>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    case 4: return dispatch_q4<4>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    case 5: return dispatch_q4<5>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    case 6: return dispatch_q4<6>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    case 7: return dispatch_q4<7>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
    case 8: return dispatch_q4<8>(qs, d, N, K, X, ldx, Xq, Y, ldy, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mmv
