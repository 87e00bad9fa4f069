/*
 * oracle.c -- plain CPU reference for the decode matrix-vector path.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Built with gcc -O2
 * -ffp-contract=off and no fast-math, so every fp32 operation written here
 * is one IEEE operation with round-to-nearest-even.
 *
 * How each part is pinned (tests/test_oracle_*.py, CPU only):
 *  - fp16 / bf16 conversion: against numpy's and torch's converters on every
 *    fp16 value, on all halfway cases and on random fp32.
 *  - Q8_1: integer-valued blocks with +-127 present (d = 1, q = x, s = sum),
 *    all-zero blocks, single non-zero, half-away rounding at exact .5,
 *    the round-trip error bound, and a printed worked example
 *    (tests/golden/q8_1_worked_example.txt, derived by hand).
 *  - BF16 GEMV: numpy float64 matmul of the widened matrix; integer pins.
 *  - Q4_0 GEMV: unit-scale integer pins against integer matmul (catches
 *    nibble order and the -8 offset), power-of-two scale pins, numpy dense
 *    dequantized matmul.
 *  - Router / top-k / weights: numpy matmul; a stable sort on
 *    (-value, index); closed forms (all-equal logits give 1/k each).
 *  - Gather lists: Python sorted() over (expert, b, j).
 *  - MoE layer: a dense numpy restatement on tiny exact cases, single-expert
 *    and identical-expert reductions, zero-weight cases.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* IEEE binary16 from binary32, round to nearest, ties to even, with
 * subnormal results, overflow to infinity and quiet NaN. */
uint16_t orc_f32_to_f16(float x) {
  uint32_t u = f32_bits(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t exp = (u >> 23) & 0xFFu;
  uint32_t man = u & 0x7FFFFFu;
  if (exp == 0xFFu)                                  /* inf or NaN */
    return (uint16_t)(sign | 0x7C00u | (man ? (0x200u | (man >> 13)) : 0u));
  if (exp == 0u)              /* fp32 zero/subnormal: far below 2^-25 */
    return sign;
  uint32_t m = man | 0x800000u;            /* 24-bit significand */
  int e16 = (int)exp - 127 + 15;           /* binary16 biased exponent */
  if (e16 >= 1) {
    /* normal candidate: keep 11 significant bits */
    uint32_t keep = m >> 13, rem = m & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (keep & 1u))) keep++;
    uint32_t h = ((uint32_t)e16 << 10) + keep - 0x400u;   /* carry ok */
    if (h >= 0x7C00u) h = 0x7C00u;                         /* overflow */
    return (uint16_t)(sign | h);
  }
  /* subnormal binary16: value / 2^-24 = m * 2^(exp - 126) */
  int shift = 126 - (int)exp;              /* >= 14 here */
  if (shift > 25) return sign;             /* below half the smallest step */
  uint32_t keep = m >> shift;
  uint32_t rem = m & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (keep & 1u))) keep++;
  return (uint16_t)(sign | keep);          /* keep may reach 0x400: fine */
}

float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  uint32_t exp = ((uint32_t)h >> 10) & 0x1Fu;
  uint32_t man = (uint32_t)h & 0x3FFu;
  if (exp == 0x1Fu) return bits_f32(sign | 0x7F800000u | (man << 13));
  if (exp == 0u) {
    /* zero or subnormal: man * 2^-24, exact in fp32 */
    float v = (float)man * 0x1p-24f;
    return sign ? -v : v;
  }
  return bits_f32(sign | ((exp - 15u + 127u) << 23) | (man << 13));
}

uint16_t orc_f32_to_bf16(float x) {
  uint32_t u = f32_bits(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu))
    return (uint16_t)((u >> 16) | 0x40u);             /* quiet NaN */
  uint32_t keep = u >> 16, rem = u & 0xFFFFu;
  if (rem > 0x8000u || (rem == 0x8000u && (keep & 1u))) keep++;
  return (uint16_t)keep;
}

float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

void orc_f32_to_f16_n(const float *x, uint16_t *h, long n) {
  for (long i = 0; i < n; i++) h[i] = orc_f32_to_f16(x[i]);
}
void orc_f16_to_f32_n(const uint16_t *h, float *x, long n) {
  for (long i = 0; i < n; i++) x[i] = orc_f16_to_f32(h[i]);
}
void orc_f32_to_bf16_n(const float *x, uint16_t *h, long n) {
  for (long i = 0; i < n; i++) h[i] = orc_f32_to_bf16(x[i]);
}
void orc_bf16_to_f32_n(const uint16_t *h, float *x, long n) {
  for (long i = 0; i < n; i++) x[i] = orc_bf16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------ */
/* dense BF16 GEMV  [STRATA: Pass 3 item 2, y = W x for one token]           */
/* ------------------------------------------------------------------------ */

void orc_gemv_bf16(const uint16_t *W, int N, int K, long ldw,
                   const float *X, long ldx, int B, double *Y) {
  for (int b = 0; b < B; b++)
    for (int n = 0; n < N; n++) {
      double acc = 0.0;
      for (int k = 0; k < K; k++)
        acc += (double)orc_bf16_to_f32(W[(long)n * ldw + k]) *
               (double)X[(long)b * ldx + k];
      Y[(long)b * N + n] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Q8_1 quantization  [FOURTEEN: kernel-class table, quantize_q8_1;          */
/*                     Eight levers, Q8 epilogue]                            */
/* ------------------------------------------------------------------------ */

void orc_quantize_q8_1(const float *X, int K, long ldx, int B,
                       int8_t *q, uint16_t *ds) {
  int nb = K / 32;
  for (int b = 0; b < B; b++)
    for (int j = 0; j < nb; j++) {
      const float *x = X + (long)b * ldx + 32L * j;
      int8_t *qq = q + (long)b * K + 32L * j;
      uint16_t *pd = ds + ((long)b * nb + j) * 2;
      float amax = 0.0f;
      for (int i = 0; i < 32; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
      }
      float d32 = amax / 127.0f;
      uint16_t d16 = orc_f32_to_f16(d32);
      if ((d16 & 0x7FFFu) == 0u) {       /* scale rounds to zero in fp16 */
        for (int i = 0; i < 32; i++) qq[i] = 0;
        pd[0] = 0; pd[1] = 0;
        continue;
      }
      float id = 1.0f / d32;
      int sum = 0;
      for (int i = 0; i < 32; i++) {
        float v = roundf(x[i] * id);          /* halves away from zero */
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        qq[i] = (int8_t)(int)v;
        sum += qq[i];
      }
      pd[0] = d16;
      pd[1] = orc_f32_to_f16(d32 * (float)sum);
    }
}

/* ------------------------------------------------------------------------ */
/* Q4_0 x Q8_1  [FOURTEEN: warp_coop Q4_0 and mul_mat_id rows;               */
/*               STRIX: split-nibble layout in the Q4_0 loaders]             */
/* ------------------------------------------------------------------------ */

static int q4_code(const uint8_t *blk, int i) {
  return i < 16 ? (blk[i] & 0x0F) : (blk[i - 16] >> 4);
}

void orc_q4_0_block_sums(const uint8_t *qs, int N, int K,
                         const int8_t *xq, int B, int32_t *I) {
  int nb = K / 32;
  for (int b = 0; b < B; b++)
    for (int n = 0; n < N; n++)
      for (int j = 0; j < nb; j++) {
        const uint8_t *blk = qs + ((long)n * nb + j) * 16;
        const int8_t *xb = xq + (long)b * K + 32L * j;
        int32_t acc = 0;
        for (int i = 0; i < 32; i++) acc += (q4_code(blk, i) - 8) * xb[i];
        I[((long)b * N + n) * nb + j] = acc;
      }
}

void orc_gemv_q4_0(const uint8_t *qs, const uint16_t *dw, int N, int K,
                   const int8_t *xq, const uint16_t *xds, int B, double *Y) {
  int nb = K / 32;
  for (int b = 0; b < B; b++)
    for (int n = 0; n < N; n++) {
      double acc = 0.0;
      for (int j = 0; j < nb; j++) {
        const uint8_t *blk = qs + ((long)n * nb + j) * 16;
        const int8_t *xb = xq + (long)b * K + 32L * j;
        long isum = 0;
        for (int i = 0; i < 32; i++) isum += (q4_code(blk, i) - 8) * xb[i];
        double dwv = orc_f16_to_f32(dw[(long)n * nb + j]);
        double dxv = orc_f16_to_f32(xds[((long)b * nb + j) * 2]);
        acc += dwv * dxv * (double)isum;
      }
      Y[(long)b * N + n] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* router, top-k, weights  [FOURTEEN: F32 router, top-k routing;             */
/*                          Four levers that did not work, F16 router]       */
/* ------------------------------------------------------------------------ */

void orc_router_logits(const float *R, int E, int H, const float *X, long ldx,
                       int B, double *logits) {
  for (int b = 0; b < B; b++)
    for (int e = 0; e < E; e++) {
      double acc = 0.0;
      for (int h = 0; h < H; h++)
        acc += (double)R[(long)e * H + h] * (double)X[(long)b * ldx + h];
      logits[(long)b * E + e] = acc;
    }
}

void orc_gemv_q4_0_f32(const uint8_t *qs, const uint16_t *dw, int N, int K,
                       const float *X, long ldx, int B, double *Y) {
  int nb = K / 32;
  for (int b = 0; b < B; b++)
    for (int n = 0; n < N; n++) {
      double acc = 0.0;
      for (int j = 0; j < nb; j++) {
        const uint8_t *blk = qs + ((long)n * nb + j) * 16;
        const float *xb = X + (long)b * ldx + 32L * j;
        double s = 0.0;
        for (int i = 0; i < 32; i++) s += (double)(q4_code(blk, i) - 8) * (double)xb[i];
        acc += (double)orc_f16_to_f32(dw[(long)n * nb + j]) * s;
      }
      Y[(long)b * N + n] = acc;
    }
}

void orc_argmax(const float *Y, long ldy, int N, int B, int32_t *ids) {
  for (int b = 0; b < B; b++) {
    const float *y = Y + (long)b * ldy;
    int best = 0;
    for (int n = 1; n < N; n++)          /* ascending scan, strict '>' */
      if (y[n] > y[best]) best = n;
    ids[b] = best;
  }
}

void orc_topk(const float *L, int E, long ldl, int B, int k, int32_t *ids) {
  char *taken = (char *)calloc((size_t)E, 1);
  for (int b = 0; b < B; b++) {
    memset(taken, 0, (size_t)E);
    const float *l = L + (long)b * ldl;
    for (int j = 0; j < k; j++) {
      int best = -1;
      for (int e = 0; e < E; e++) {      /* ascending scan, strict '>' */
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[(long)b * k + j] = best;
    }
  }
  free(taken);
}

void orc_gate_weights(const double *logits, long ldl, const int32_t *ids,
                      int B, int k, double *w) {
  for (int b = 0; b < B; b++) {
    const double *l = logits + (long)b * ldl;
    const int32_t *id = ids + (long)b * k;
    double m = l[id[0]];
    for (int j = 1; j < k; j++) if (l[id[j]] > m) m = l[id[j]];
    double den = 0.0;
    for (int j = 0; j < k; j++) den += exp(l[id[j]] - m);
    for (int j = 0; j < k; j++) w[(long)b * k + j] = exp(l[id[j]] - m) / den;
  }
}

int orc_gather(const int32_t *ids, int B, int k, int32_t *unique,
               int32_t *offsets, int32_t *pairs) {
  int total = B * k, U = 0, filled = 0;
  /* plain selection: repeatedly take the smallest expert id not yet listed */
  int prev = -1;
  for (;;) {
    int next = -1;
    for (int t = 0; t < total; t++)
      if (ids[t] > prev && (next < 0 || ids[t] < next)) next = ids[t];
    if (next < 0) break;
    unique[U] = next;
    offsets[U] = filled;
    for (int t = 0; t < total; t++)          /* t = b*k + j ascending */
      if (ids[t] == next) pairs[filled++] = t;
    U++;
    prev = next;
  }
  offsets[U] = filled;
  return U;
}

/* ------------------------------------------------------------------------ */
/* MoE layer  [FOURTEEN: mul_mat_id expert matvecs, Q8 epilogue in the gated */
/*             kernel, four rows per wave down projection, router with 257   */
/*             rows (shared expert)]                                         */
/* ------------------------------------------------------------------------ */

void orc_moe_route(const orc_moe *L, const float *X, long ldx, int B,
                   double *logits, int32_t *ids, double *w, double *s) {
  int E = L->E, k = L->k;
  orc_router_logits(L->router, E, L->H, X, ldx, B, logits);
  /* the selection decision is taken on fp32 logits */
  float *lf = (float *)malloc(sizeof(float) * (size_t)B * E);
  for (long i = 0; i < (long)B * E; i++) lf[i] = (float)logits[i];
  orc_topk(lf, E, E, B, k, ids);
  free(lf);
  orc_gate_weights(logits, E, ids, B, k, w);
  for (int b = 0; b < B; b++) {
    if (!L->shared_gate_row) { s[b] = 1.0; continue; }
    double z = 0.0;
    for (int h = 0; h < L->H; h++)
      z += (double)L->shared_gate_row[h] * (double)X[(long)b * ldx + h];
    s[b] = 1.0 / (1.0 + exp(-z));
  }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

void orc_moe_gate_up(const orc_moe *L, const float *X, long ldx, int B,
                     const int32_t *ids, float *h) {
  int H = L->H, I = L->I, k = L->k, nbh = H / 32;
  int8_t *xq = (int8_t *)malloc((size_t)H);
  uint16_t *xds = (uint16_t *)malloc(sizeof(uint16_t) * 2 * (size_t)nbh);
  double *g = (double *)malloc(sizeof(double) * (size_t)I);
  double *u = (double *)malloc(sizeof(double) * (size_t)I);
  int npairs = B * k + (L->sh_gate_qs ? B : 0);
  for (int p = 0; p < npairs; p++) {
    int b = p < B * k ? p / k : p - B * k;
    const uint8_t *gq, *uq; const uint16_t *gd, *ud;
    if (p < B * k) {
      long e = ids[p];
      gq = L->gate_qs + e * I * nbh * 16; gd = L->gate_d + e * I * nbh;
      uq = L->up_qs + e * I * nbh * 16;   ud = L->up_d + e * I * nbh;
    } else {
      gq = L->sh_gate_qs; gd = L->sh_gate_d; uq = L->sh_up_qs; ud = L->sh_up_d;
    }
    orc_quantize_q8_1(X + (long)b * ldx, H, ldx, 1, xq, xds);
    orc_gemv_q4_0(gq, gd, I, H, xq, xds, 1, g);
    orc_gemv_q4_0(uq, ud, I, H, xq, xds, 1, u);
    for (int n = 0; n < I; n++) h[(long)p * I + n] = (float)(silu(g[n]) * u[n]);
  }
  free(xq); free(xds); free(g); free(u);
}

void orc_moe_down(const orc_moe *L, const int8_t *hq, const uint16_t *hds,
                  int B, const int32_t *ids, const double *w, const double *s,
                  double *Y) {
  int H = L->H, I = L->I, k = L->k, nbi = I / 32;
  double *t = (double *)malloc(sizeof(double) * (size_t)H);
  for (long i = 0; i < (long)B * H; i++) Y[i] = 0.0;
  for (int b = 0; b < B; b++) {
    for (int j = 0; j <= k; j++) {
      const uint8_t *dq; const uint16_t *dd; double wt; int p;
      if (j < k) {
        long e = ids[b * k + j];
        dq = L->down_qs + e * H * nbi * 16; dd = L->down_d + e * H * nbi;
        wt = w[b * k + j]; p = b * k + j;
      } else {
        if (!L->sh_down_qs) break;
        dq = L->sh_down_qs; dd = L->sh_down_d; wt = s[b]; p = B * k + b;
      }
      orc_gemv_q4_0(dq, dd, H, I, hq + (long)p * I, hds + (long)p * nbi * 2,
                    1, t);
      for (int n = 0; n < H; n++) Y[(long)b * H + n] += wt * t[n];
    }
  }
  free(t);
}

void orc_moe_layer(const orc_moe *L, const float *X, long ldx, int B,
                   int32_t *ids, double *w, double *s, float *h, double *Y) {
  int E = L->E, k = L->k, I = L->I;
  int npairs = B * k + (L->sh_gate_qs ? B : 0);
  double *lg = (double *)malloc(sizeof(double) * (size_t)B * E);
  int32_t *id = ids ? ids : (int32_t *)malloc(sizeof(int32_t) * (size_t)B * k);
  double *ww = w ? w : (double *)malloc(sizeof(double) * (size_t)B * k);
  double *ss = s ? s : (double *)malloc(sizeof(double) * (size_t)B);
  float *hh = h ? h : (float *)malloc(sizeof(float) * (size_t)npairs * I);
  int8_t *hq = (int8_t *)malloc((size_t)npairs * I);
  uint16_t *hds = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)npairs * (I / 32) * 2);
  orc_moe_route(L, X, ldx, B, lg, id, ww, ss);
  orc_moe_gate_up(L, X, ldx, B, id, hh);
  orc_quantize_q8_1(hh, I, I, npairs, hq, hds);
  orc_moe_down(L, hq, hds, B, id, ww, ss, Y);
  free(lg); free(hq); free(hds);
  if (!ids) free(id);
  if (!w) free(ww);
  if (!s) free(ss);
  if (!h) free(hh);
}
