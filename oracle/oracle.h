/*
 * oracle.h -- plain, slow CPU reference for the decode matrix-vector path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no source with the HIP
 * library (moe_matvec_amd/csrc) and neither side includes the other.
 *
 * Every function restates a definition in the plainest form: straight loops,
 * float64 accumulation wherever the definition is a real-valued sum, and
 * fp32 arithmetic only where the definition itself fixes fp32 (the Q8_1
 * quantizer, and the fp32 logits on which the top-k decision is taken).
 *
 * Sources (web pages, cited by title and section):
 *  [STRATA]  "Beating llama.cpp from Scratch on Consumer AMD: Building Strata"
 *            -- The Optimization Passes, Pass 3 item 2 (custom BF16 GEMV for
 *            single-token decode); Act 6 (the memory-bandwidth wall).
 *  [FOURTEEN] "Fourteen hours to 100 tokens per second"
 *            -- "The trace that changed everything" (kernel-class table:
 *            mul_mat_id expert matvecs, warp_coop Q4_0 dense matvecs,
 *            quantize_q8_1, F32 router, top-k routing); "Eight levers that
 *            worked" (four rows per wave for K <= 512, Q8 epilogue in the
 *            gated kernel); "The router with 257 rows" (shared expert,
 *            sigmoid weight); "Four levers that did not work" (F16 router
 *            changed tie outcomes, so the router stays F32).
 *  [STRIX]   "Flash-Next on Strix Halo" -- Correctness fixes (split-nibble
 *            Q4_0 loader layout); Expert GEMMs (per-expert row lists).
 *
 * Where the pages name a format or step without defining it numerically,
 * the reading taken is stated at the function.
 *
 * Parity pins: every function here is pinned by CPU tests in tests/ against
 * closed forms, brute force or independent library routines (numpy); see the
 * header comment of oracle.c for the list.
 */
#ifndef MMV_ORACLE_H
#define MMV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ---------------------------------------------------- */
uint16_t orc_f32_to_f16(float x);   /* IEEE binary16, round to nearest even */
float    orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float x);  /* bfloat16, round to nearest even      */
float    orc_bf16_to_f32(uint16_t h);
void orc_f32_to_f16_n(const float *x, uint16_t *h, long n);
void orc_f16_to_f32_n(const uint16_t *h, float *x, long n);
void orc_f32_to_bf16_n(const float *x, uint16_t *h, long n);
void orc_bf16_to_f32_n(const uint16_t *h, float *x, long n);

/* ---- dense BF16 GEMV ----------------------------------------------------
 * Y[b*N + n] = sum_k bf16(W[n*ldw + k]) * X[b*ldx + k], in float64. */
void orc_gemv_bf16(const uint16_t *W, int N, int K, long ldw,
                   const float *X, long ldx, int B, double *Y);

/* ---- Q8_1 activation quantization ---------------------------------------
 * Planar Q8_1 for B rows of K (K % 32 == 0):
 *   q  : int8  [B][K]           codes
 *   ds : fp16  [B][K/32][2]     {d, s} per block
 * Per block of 32 values x_i:
 *   amax = max |x_i|;  d32 = amax / 127 (fp32 division)
 *   if fp16(d32) == 0: d = s = 0, q_i = 0   (scale not representable)
 *   else id = 1 / d32 (fp32), q_i = clamp(roundf(x_i * id), -127, 127)
 *        d = fp16(d32),  s = fp16(d32 * (float) sum_i q_i)
 */
void orc_quantize_q8_1(const float *X, int K, long ldx, int B,
                       int8_t *q, uint16_t *ds);

/* ---- Q4_0 x Q8_1 GEMV ---------------------------------------------------
 * Q4_0 matrix N x K, planar: qs [N][K/32][16] bytes, d fp16 [N][K/32].
 * Block byte i holds code i in the low nibble and code i+16 in the high
 * nibble (split-nibble); weight = d * (code - 8).
 * I[(b*N + n)*nb + j] = sum_i (code_i - 8) * q_x[b][32j + i]   (exact int)
 * Y[b*N + n] = sum_j f16(d_w) * f16(d_x) * I, in float64. */
void orc_q4_0_block_sums(const uint8_t *qs, int N, int K,
                         const int8_t *xq, int B, int32_t *I);
void orc_gemv_q4_0(const uint8_t *qs, const uint16_t *dw, int N, int K,
                   const int8_t *xq, const uint16_t *xds, int B, double *Y);

/* ---- Q4_0 weights x fp32 activations (W4A16: no Q8_1 step) -------------
 * Y[b*N + n] = sum_j f16(d_w[n][j]) * sum_i (code_i - 8) * X[b*ldx + 32j + i],
 * in float64.  [STRATA: "BF16 vs Quantization" (W4A16 INT4), and the
 * dequant-gemv kernels its closing paragraph announces] */
void orc_gemv_q4_0_f32(const uint8_t *qs, const uint16_t *dw, int N, int K,
                       const float *X, long ldx, int B, double *Y);

/* ---- argmax of rows (the top-1 case of orc_topk) ------------------------
 * ids[b] = the index of the largest Y[b*ldy + n], n < N (fp32 compare, so
 * -0 == +0); among equal values the lowest index.  [STRATA: The
 * Optimization Passes, Pass 3 item 3: on-device argmax over the logits] */
void orc_argmax(const float *Y, long ldy, int N, int B, int32_t *ids);

/* ---- F32 router, top-k, renormalised gate weights ----------------------- */
/* logits[b*E + e] = sum_h R[e*H + h] * X[b*ldx + h], in float64 */
void orc_router_logits(const float *R, int E, int H, const float *X, long ldx,
                       int B, double *logits);
/* ids[b*k + j]: the k largest of the fp32 logits L[b*ldl + e], in descending
 * order; among equal values the lower index ranks first. */
void orc_topk(const float *L, int E, long ldl, int B, int k, int32_t *ids);
/* w[b*k + j] = exp(l_j - m) / sum_j' exp(l_j' - m) over the selected ids,
 * m = max selected logit; logits in float64, row stride ldl. */
void orc_gate_weights(const double *logits, long ldl, const int32_t *ids,
                      int B, int k, double *w);
/* gather lists: U unique experts ascending, offsets[U+1], pairs = b*k + j
 * grouped by expert, then b, then j.  Returns U. */
int orc_gather(const int32_t *ids, int B, int k, int32_t *unique,
               int32_t *offsets, int32_t *pairs);

/* ---- MoE layer ---------------------------------------------------------- */
typedef struct {
  int E, H, I, k;
  const float *router;            /* E x H fp32                              */
  const float *shared_gate_row;   /* H fp32 or NULL (shared weight = 1)      */
  const uint8_t *gate_qs, *up_qs, *down_qs;     /* stacked, expert-major     */
  const uint16_t *gate_d, *up_d, *down_d;       /* gate/up I x H, down H x I */
  const uint8_t *sh_gate_qs, *sh_up_qs, *sh_down_qs;  /* NULL: no shared    */
  const uint16_t *sh_gate_d, *sh_up_d, *sh_down_d;
} orc_moe;

/* Routing: logits (B x E, float64), ids (B x k), w (B x k), s (B). */
void orc_moe_route(const orc_moe *L, const float *X, long ldx, int B,
                   double *logits, int32_t *ids, double *w, double *s);
/* Gate/up stage for every (row, slot) pair p = b*k + j and, when the layer
 * has a shared expert, p = B*k + b:  h[p*I + n] = fp32(silu(g_n) * u_n)
 * with g, u the Q4_0 x Q8_1(x_b) products of the pair's expert. */
void orc_moe_gate_up(const orc_moe *L, const float *X, long ldx, int B,
                     const int32_t *ids, float *h);
/* Down stage from quantized h (planar Q8_1 with B*k (+B) rows of I):
 * Y[b*H + n] = sum_j w_bj * down_{e_bj}(h_p) + s_b * down_shared(h_p'). */
void orc_moe_down(const orc_moe *L, const int8_t *hq, const uint16_t *hds,
                  int B, const int32_t *ids, const double *w, const double *s,
                  double *Y);
/* Whole layer: route, gate/up, Q8_1(h), down.  Outputs may be NULL except Y. */
void orc_moe_layer(const orc_moe *L, const float *X, long ldx, int B,
                   int32_t *ids, double *w, double *s, float *h, double *Y);

#ifdef __cplusplus
}
#endif
#endif
