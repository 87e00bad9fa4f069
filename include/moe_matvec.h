/*
 * moe_matvec.h -- C ABI of the decode matrix-vector library for AMD Instinct
 * MI355X (CDNA4, gfx950).
 *
 * The library computes the products that dominate single-token (and up to
 * 8-row) LLM decode, y = W x, streaming every weight byte once per call:
 * dense BF16 GEMV, Q4_0 x Q8_1 GEMV with on-the-fly activation quantization,
 * and the mixture-of-experts path (F32 router, softmax, top-k, gathered
 * per-expert gate/up/down products, shared expert).
 *
 * Sources (web pages, cited by title and section):
 *  [STRATA]   "Beating llama.cpp from Scratch on Consumer AMD: Building
 *             Strata" -- The Optimization Passes, Pass 3 (HIP graph replay;
 *             custom vectorized BF16 GEMV for M = 1); The Kernel Execution
 *             Profile (GEMV share of decode; the memory-bandwidth wall).
 *  [FOURTEEN] "Fourteen hours to 100 tokens per second" -- kernel-class table
 *             in "The trace that changed everything"; "Eight levers that
 *             worked"; "The router with 257 rows"; "Four levers that did not
 *             work"; "Two bugs nobody was looking for".
 *  [STRIX]    "Flash-Next on Strix Halo" -- Expert GEMMs (per-expert row
 *             lists); Correctness fixes (split-nibble Q4_0 loaders).
 *
 * Conventions for every entry point
 *  - Matrices are N x K (out x in), row-major: y[b][n] = sum_k W[n][k] x[b][k].
 *  - B is the number of activation rows (tokens), 1 <= B <= MMV_MAX_BATCH.
 *  - All tensor pointers are DEVICE pointers owned by the caller.  `stream`
 *    is a hipStream_t passed as void* (NULL = the default stream).
 *  - Calls only enqueue work on `stream`: they never allocate, free,
 *    synchronize or read device memory on the host, so they can be captured
 *    in a HIP graph.  Outputs are fully overwritten, never accumulated.
 *  - Every argument check runs on the host before any launch; a negative
 *    return means nothing was enqueued.  MMV_E_HIP reports a failed launch
 *    (see mmv_last_hip_error).  Faults inside a kernel surface at the
 *    caller's next synchronization.
 *  - Results are deterministic: no floating-point atomics; repeated calls
 *    on the same inputs give bit-identical outputs.  Each row of a B-row
 *    call equals the 1-row call on that row, bit for bit, for
 *    quantize_q8_1, argmax_rows and the MoE calls.  The GEMVs switch to the
 *    matrix cores at some B, and each kernel sums in its own order: rows
 *    are bit-identical across the B one kernel serves and agree within
 *    rounding across kernels.  gemv_bf16: B = 1 (fp32 fused multiply-adds)
 *    against B >= 2 (x split into bf16 high + low parts).  gemv_q4_0 at
 *    K <= 4096: B <= 2 against B >= 3 for fp32 x, B <= 4 against B >= 5
 *    for a Q8_1 buffer (the exact block integers are the same).
 *    gemv_q4_0_f32 at K <= 4096: B = 1 against B >= 2.
 *  - Outputs must not overlap inputs (MMV_E_ALIAS).
 *
 * Data formats
 *  - BF16 weights: uint16 bit patterns of bfloat16.
 *  - Q4_0 matrix (planar): blocks of 32 consecutive weights of one row.
 *      qs : uint8  [N][K/32][16]  block byte i = code[i] | code[i+16] << 4
 *                                  (split-nibble), codes 0..15
 *      d  : fp16   [N][K/32]      block scale
 *    weight = d * (code - 8).  The 16 code bytes of a block are one aligned
 *    128-bit word; the scales sit in their own plane.
 *  - Q8_1 activations (planar), B rows of K, K % 32 == 0, one buffer of
 *    mmv_q8_1_bytes(K, B) bytes:
 *      bytes [0, B*K)                 int8 codes, row-major [B][K]
 *      bytes [B*K, B*K + 4*B*K/32)    fp16 pairs {d, s} per block [B][K/32]
 *    Per block of 32 values x_i:  amax = max|x_i|, d32 = amax / 127 (fp32);
 *    if fp16(d32) == 0 the block is all zero (d = s = 0, codes 0); else
 *    q_i = clamp(roundf(x_i * (1/d32)), -127, 127) with roundf rounding
 *    halves away from zero, d = fp16(d32), s = fp16(d32 * sum_i q_i).
 *    Inputs must be finite.
 */
#ifndef MOE_MATVEC_H
#define MOE_MATVEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MMV_MAX_BATCH   8     /* rows per call                              */
#define MMV_MOE_MAX_BATCH 64  /* rows per MoE call (verify / prefill batches) */
#define MMV_MAX_EXPERTS 1024  /* router rows E                              */
#define MMV_MAX_TOPK    16    /* experts per row k                          */
#define MMV_Q4_MAX_XK   49152 /* B*K limit of gemv_q4_0 (x staged in LDS)   */
#define MMV_Q4F32_MAX_XK 36864 /* B*K limit of gemv_q4_0_f32 (fp32 x in LDS) */

typedef enum {
  MMV_OK = 0,
  MMV_E_NULL = -1,      /* a required pointer is NULL                       */
  MMV_E_SHAPE = -2,     /* a size is out of range or not a block multiple   */
  MMV_E_ALIGN = -3,     /* a pointer or leading dimension is misaligned     */
  MMV_E_BATCH = -4,     /* B outside 1..MMV_MAX_BATCH (MoE: MMV_MOE_MAX_BATCH) */
  MMV_E_TOPK = -5,      /* k outside 1..min(E, MMV_MAX_TOPK)                 */
  MMV_E_WORKSPACE = -6, /* workspace NULL or smaller than required          */
  MMV_E_ALIAS = -7,     /* an output overlaps an input                      */
  MMV_E_HIP = -8,       /* the HIP runtime rejected a launch                */
  MMV_E_ARG = -9        /* inconsistent arguments (e.g. both X and Xq)      */
} mmv_status;

/* Human-readable text for a status code (static storage). */
const char *mmv_status_str(int status);
/* hipError_t of the last MMV_E_HIP on the calling thread (0 if none). */
int mmv_last_hip_error(void);

/* Q4_0 matrix descriptor (planar layout above).  qs 16-byte aligned,
 * d 2-byte aligned, K % 32 == 0. */
typedef struct {
  const uint8_t *qs;
  const uint16_t *d;
  int32_t N;
  int32_t K;
} mmv_q4_0;

/* Size in bytes of a planar Q8_1 buffer for B rows of K. */
size_t mmv_q8_1_bytes(int32_t K, int32_t B);

/* --------------------------------------------------------------------------
 * gemv_bf16 -- dense BF16 GEMV.  [STRATA: Pass 3 item 2]
 *   Y[b*ldy + n] = sum_k bf16(W[n*ldw + k]) * X[b*ldx + k]   (fp32 accumulate)
 *   W: N x K bf16, rows 16-byte aligned (W 16-byte aligned, ldw % 8 == 0,
 *      ldw >= K); K % 8 == 0.  Gate and up projections stored as one
 *      [2I x H] matrix are one call.
 *   X: B x K fp32, 16-byte aligned, ldx % 4 == 0, ldx >= K.
 *   Y: B x N fp32, ldy >= N.
 * ------------------------------------------------------------------------ */
int gemv_bf16(const uint16_t *W, int32_t N, int32_t K, int64_t ldw,
              const float *X, int64_t ldx, int32_t B,
              float *Y, int64_t ldy, void *stream);

/* --------------------------------------------------------------------------
 * quantize_q8_1 -- fp32 activations to planar Q8_1.
 *   [FOURTEEN: kernel-class table, "Activation quantization (quantize_q8_1)"]
 *   X: B x K fp32 (K % 32 == 0, 16-byte aligned, ldx % 4 == 0).
 *   Xq: mmv_q8_1_bytes(K, B) bytes, 16-byte aligned.
 *   The same device routine quantizes inside gemv_q4_0 and moe_mul_mat_id,
 *   so their codes are identical to this call's.
 * ------------------------------------------------------------------------ */
int quantize_q8_1(const float *X, int32_t K, int64_t ldx, int32_t B,
                  void *Xq, void *stream);

/* --------------------------------------------------------------------------
 * gemv_q4_0 -- Q4_0 weights x Q8_1 activations.
 *   [FOURTEEN: "Dense matvecs (warp_coop Q4_0)"; four rows per wave for
 *    K <= 512 in "Eight levers that worked"]
 *   Y[b*ldy + n] = sum_j d_w[n][j] * d_x[b][j] * I[b][n][j],
 *   I[b][n][j] = sum_i (code_i - 8) * q_x[b][32j + i]  (exact int32), then
 *   fp32 scaling and sums.  K <= 4096 with B >= 3 (fp32 x) or B >= 5 (a
 *   Q8_1 buffer) runs on the int8 matrix cores, the rest on dot4 kernels;
 *   the two sum the blocks in different orders, so rows agree within
 *   rounding (rel-L2 ~1e-7) across them and bit for bit within each.
 *   Activations, one of three ways (the codes are bit-identical in all):
 *     X only:  fp32 B x K, quantized to Q8_1 inside every workgroup (one
 *              launch; the better choice at B = 1, and at B = 3 to 5 with
 *              K <= 4096, where the matrix cores quantize x once per CU);
 *     Xq only: planar Q8_1 of B rows of K, read as given;
 *     both:    X is first quantized into the caller's Xq buffer
 *              (mmv_q8_1_bytes(K, B) bytes, an output, left holding
 *              Q8_1(X)), then the product reads Xq (two launches; the
 *              better choice from B = 6, and at any B >= 2 with K > 4096,
 *              where repeating the quantization in every workgroup costs
 *              more than the extra launch).
 *   X only and Xq give bit-identical rows where they take the same kernel
 *   (B <= 2, B >= 5 or K > 4096).
 *   B*K <= MMV_Q4_MAX_XK.  Y: B x N fp32, ldy >= N.
 * ------------------------------------------------------------------------ */
int gemv_q4_0(const mmv_q4_0 *W, const float *X, int64_t ldx, const void *Xq,
              int32_t B, float *Y, int64_t ldy, void *stream);

/* --------------------------------------------------------------------------
 * gemv_q4_0_f32 -- Q4_0 weights x fp32 activations (W4A16: no Q8_1 step).
 *   [STRATA: "BF16 vs Quantization" (W4A16 INT4 with on-the-fly
 *    dequantization) and the dequant-gemv kernels its closing paragraph
 *    announces]
 *   Y[b*ldy + n] = sum_j d_w[n][j] * sum_i (code_i - 8) * X[b*ldx + 32j + i],
 *   fp32 sums.  x is split into bf16 hi + lo (x kept to 2^-17 relative) and
 *   each code enters as bf16 128 + code, so every product is exact; per
 *   block d_w * (sum_i (128 + code_i) (hi_i + lo_i) - 136 * sum_i (hi_i +
 *   lo_i)).  B = 1 or K > 4096: two codes per v_dot2 (fp32 accumulation);
 *   B >= 2 with K <= 4096: the matrix cores.  The two agree within rounding
 *   (rel-L2 ~1e-5), and each is bit-identical across the B it serves.
 *   Any K % 32 == 0 with B * K <= MMV_Q4F32_MAX_XK (x of every row is
 *   staged in on-chip memory: B = 8 at K = 4096, B = 3 at K = 11008,
 *   B = 1 up to K = 36864).
 *   X: B x K fp32, 16-byte aligned, ldx % 4 == 0.  Y: B x N fp32, ldy >= N.
 * ------------------------------------------------------------------------ */
int gemv_q4_0_f32(const mmv_q4_0 *W, const float *X, int64_t ldx, int32_t B,
                  float *Y, int64_t ldy, void *stream);

/* --------------------------------------------------------------------------
 * argmax_rows -- per row, the index of the largest value, on the device.
 *   [STRATA: The Optimization Passes, Pass 3 item 3: argmax of the
 *    248,320 logits on the device, 4 bytes per token to the host]
 *   ids[b] = index of the largest Y[b*ldy + n], n < N; equal values rank
 *   by lower index and -0 equals +0 (the ordering of moe_route_topk).
 *   vals[b] (optional, may be NULL) = that value.  Y finite, 4-byte
 *   aligned, ldy >= N.  workspace: mmv_argmax_workspace_bytes(N, B) bytes,
 *   8-byte aligned, no initialisation needed.  Two launches.
 * ------------------------------------------------------------------------ */
size_t mmv_argmax_workspace_bytes(int32_t N, int32_t B);
int argmax_rows(const float *Y, int64_t ldy, int32_t N, int32_t B, int32_t *ids,
                float *vals, void *workspace, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * moe_route_topk -- F32 router, softmax, top-k, renormalised gate weights.
 *   [FOURTEEN: "F32 router (mul_mat_vec_f)", "Top-k routing"; the F16
 *    router was rejected because ties broke differently; "The router with
 *    257 rows": top-k writes ids and weights straight into the buffers the
 *    expert products read]
 *   router: E x H fp32 (16-byte aligned, H % 4 == 0), or NULL: then X holds
 *           B rows of E logits (ldx >= E) and the matvec is skipped.
 *   logits: B x (E+1) fp32 output: logits[b*(E+1) + e]; column E holds the
 *           shared-gate logit when shared_gate_row != NULL.
 *   ids:    B x k int32: the k largest logits of row b, in descending
 *           order; equal logits rank by lower expert index.
 *   weights:B x k fp32: softmax over all E renormalised over the selected
 *           k, i.e. exp(l_j - l_max) / sum over selected.
 *   shared_w: B fp32 (may be NULL): sigmoid(shared_gate_row . x_b), or 1
 *           when shared_gate_row is NULL.
 *   1 <= k <= min(E, MMV_MAX_TOPK), E <= MMV_MAX_EXPERTS,
 *   1 <= B <= MMV_MOE_MAX_BATCH.
 * ------------------------------------------------------------------------ */
int moe_route_topk(const float *router, int32_t E, int32_t H,
                   const float *X, int64_t ldx, int32_t B, int32_t k,
                   const float *shared_gate_row, float *logits,
                   int32_t *ids, float *weights, float *shared_w,
                   void *stream);

/* One MoE layer's weights.  Routed experts are stacked expert-major, as in
 * a stacked expert tensor of the model file [FOURTEEN: "The router with 257
 * rows": the experts of a layer as one stacked tensor, the shared expert
 * beside it]: expert e's gate block (i, j) is at
 * gate_qs + e*gate_qs_stride + (i*(H/32) + j)*16 and
 * gate_d[e*gate_d_stride + i*(H/32) + j]; up likewise; down is H x I per
 * expert.  A zero stride means contiguous experts (qs: I*H/2 bytes, d:
 * I*H/32 elements, for all three matrices).  A nonzero qs stride is a
 * multiple of 16 bytes and at least I*H/2; a nonzero d stride is at least
 * I*H/32 (else MMV_E_SHAPE).  The shared expert has one matrix of each
 * (sh_*_qs == NULL: no shared expert).  H % 32 == 0, I % 32 == 0. */
typedef struct {
  int32_t n_experts;              /* E */
  int32_t hidden;                 /* H */
  int32_t inter;                  /* I */
  int32_t top_k;                  /* k */
  const float *router;            /* E x H fp32                              */
  const float *shared_gate_row;   /* H fp32, NULL: shared weight 1           */
  const uint8_t *gate_qs, *up_qs, *down_qs;
  const uint16_t *gate_d, *up_d, *down_d;
  const uint8_t *sh_gate_qs, *sh_up_qs, *sh_down_qs;
  const uint16_t *sh_gate_d, *sh_up_d, *sh_down_d;
  int64_t gate_qs_stride, up_qs_stride, down_qs_stride;  /* bytes, 0: contiguous  */
  int64_t gate_d_stride, up_d_stride, down_d_stride;     /* elements, 0: contiguous */
} mmv_moe_layer;

/* Optional staged outputs of moe_mul_mat_id, for tests: device buffers the
 * caller owns, each may be NULL.  P = B*k routed pairs (p = b*k + j) plus B
 * shared pairs (p = B*k + b) when the layer has a shared expert.  The Q8_1
 * buffers use the planar layout of the header (codes, then {d, s} pairs).
 * [FOURTEEN: "Two bugs nobody was looking for": quantized activations as
 *  explicit buffers, so each stage can be compared on its own] */
typedef struct {
  float *h;            /* P x I fp32: silu(gate) * up for each pair          */
  int32_t *unique;     /* [B*k]: sorted unique routed experts               */
  int32_t *offsets;    /* [B*k + 1]: pair ranges per unique expert          */
  int32_t *pairs;      /* [B*k]: b*k + j grouped by expert, then b, then j  */
  int32_t *n_unique;   /* [1]                                               */
  void *x_q8;          /* mmv_q8_1_bytes(H, B): Q8_1 of the B rows of x, as
                          the gate/up workgroups stage it (same routine)     */
  float *gate_out;     /* P x I fp32: gate product of each pair             */
  float *up_out;       /* P x I fp32: up product of each pair               */
  void *h_q8;          /* mmv_q8_1_bytes(I, P): Q8_1(h), the down input      */
  float *down_out;     /* P x H fp32: each pair's down product, before the
                          weight (0 for a pair whose id is outside [0, E))   */
} mmv_moe_debug;

/* Workspace bytes for moe_mul_mat_id / moe_layer_decode at B rows.
 * Layout: bytes [0, mmv_q8_1_bytes(I, P)) hold Q8_1(h) for the P pairs
 * (P = B*k routed pairs p = b*k + j, then B shared pairs p = B*k + b),
 * followed by the integer code sums of those blocks, the per-expert row
 * lists, the routing buffers that moe_layer_decode uses, P x H fp32
 * per-pair down products (the by-expert down projection for B >= 3), and
 * for B > 8 the gate/up work records (32 bytes per expert and 8-row group).
 * 256-byte aligned workspace required. */
size_t moe_workspace_bytes(const mmv_moe_layer *L, int32_t B);

/* --------------------------------------------------------------------------
 * moe_mul_mat_id -- routed + shared expert FFN for B rows.
 *   [FOURTEEN: "Expert matvecs (mul_mat_id)"; "Q8 epilogue in the gated
 *    kernel"; "Four rows per wave (K <= 512)" for the down projection;
 *    STRIX: per-expert row lists]
 *   For each pair (b, j) with expert e = ids[b*k + j] (and the shared
 *   expert for every row):  g = Gate_e (x) Q8_1(x_b),  u = Up_e (x) Q8_1(x_b)
 *   (Q4_0 x Q8_1 products), h = silu(g) * u in fp32, then Q8_1(h) along I,
 *   and
 *     Y[b*ldy + n] = sum_j weights[b*k+j] * (Down_e (x) Q8_1(h))[n]
 *                    + shared_w[b] * (Down_sh (x) Q8_1(h_sh))[n].
 *   Each unique expert's weights are read once for all rows that chose it.
 *   ids: B x k int32 in [0, E), distinct within a row (an id outside
 *   [0, E) adds nothing; a row naming one expert twice gets an unspecified
 *   result, every access staying in bounds); weights: B x k fp32;
 *   shared_w: B fp32 or NULL (weight 1).  X: B x H fp32, ldx % 4 == 0.
 *   Y: B x H fp32.  workspace: moe_workspace_bytes(L, B) bytes.
 *   1 <= B <= MMV_MOE_MAX_BATCH.  Verify / prefill batches (B > 8) take a
 *   row-list pass over all B*k pairs [STRIX: Expert GEMMs: per-expert row
 *   lists, then compact (expert, tile) work]; each (expert, 32-row tile)
 *   workgroup walks its rows eight at a time with the weights re-read from
 *   cache, and every row's result is the same bits as in a call of B <= 8.
 * ------------------------------------------------------------------------ */
int moe_mul_mat_id(const mmv_moe_layer *L, const float *X, int64_t ldx,
                   int32_t B, const int32_t *ids, const float *weights,
                   const float *shared_w, float *Y, int64_t ldy,
                   void *workspace, size_t ws_bytes,
                   const mmv_moe_debug *dbg, void *stream);

/* --------------------------------------------------------------------------
 * moe_layer_decode -- the whole MoE layer: the router rows; top-k with the
 *   per-expert row lists (inside every gate/up workgroup for B <= 2, in a
 *   one-workgroup kernel of its own for larger B); the gate/up of the
 *   shared and the routed experts with the Q8_1 epilogue; the down
 *   projection with the combine (one kernel for B <= 2; for B >= 3 one
 *   workgroup per (expert, 64 output rows), then a combine kernel).  Three
 *   launches for B <= 2, five for B <= 8, six above (the router, top-k,
 *   the row-list pass, gate/up per 8-row group of an expert, down,
 *   combine); with H other than 1024 or 2048 the router takes a launch per
 *   8 rows (5 + ceil(B/8) launches above B = 8).  Every row's
 *   result is the same bits whatever
 *   the other rows of the batch are.  1 <= B <= MMV_MOE_MAX_BATCH.
 *   Routing stays in device memory.  ids / weights (B x k) may be NULL;
 *   when given they receive the routing decision.  The workspace needs no
 *   initialisation; calls that share a workspace must not overlap.
 *   [STRATA: Pass 3 item 1, graph replay; FOURTEEN: launches below five
 *   microseconds cost more than they run; "The router with 257 rows"]
 * ------------------------------------------------------------------------ */
int moe_layer_decode(const mmv_moe_layer *L, const float *X, int64_t ldx,
                     int32_t B, float *Y, int64_t ldy,
                     int32_t *ids, float *weights,
                     void *workspace, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * moe_layer_decode_noalloc -- moe_layer_decode without a caller workspace,
 *   for callers that cannot allocate device memory: code under HIP graph
 *   capture, tight serving loops, harnesses that forbid hipMalloc.
 *   The same kernels and results as moe_layer_decode (bit for bit); the
 *   workspace is an array inside the library, MMV_NOALLOC_WS_BYTES bytes per
 *   GPU, held from the module load until the process ends.  The call
 *   allocates nothing.  A layer and B whose moe_workspace_bytes exceeds
 *   MMV_NOALLOC_WS_BYTES is refused with MMV_E_WORKSPACE (512 experts,
 *   H = 2048, I = 512, top-10 with a shared expert fit up to B = 64).
 *   Every call on one GPU uses that GPU's one array, which keeps the last
 *   call's contents (no call needs it cleared): calls that overlap in time
 *   on one GPU (other streams, other threads) race and must not be issued;
 *   calls ordered on one stream are fine.  The first call on each GPU looks
 *   up the array's device address (a host-side runtime query).
 * ------------------------------------------------------------------------ */
#define MMV_NOALLOC_WS_BYTES ((size_t)8 << 20)
size_t mmv_noalloc_ws_bytes(void);
int moe_layer_decode_noalloc(const mmv_moe_layer *L, const float *X, int64_t ldx,
                             int32_t B, float *Y, int64_t ldy,
                             int32_t *ids, float *weights, void *stream);

/* --------------------------------------------------------------------------
 * Measurement utility: device read-bandwidth probe.  ["hanzo-engine: A
 * Portable Single-Binary LLM Inference Engine", The Bandwidth Wall: decode
 * bandwidth is compared with a measured device roofline probe]
 *   Streams `bytes` (multiple of 16, at most 2^38; buf 16-byte aligned) with
 *   128-bit non-temporal loads, 32 KiB per one-shot workgroup, and writes
 *   one xor-fold word per wave to out[(wave index) % mmv_probe_slots()]
 *   (waves sharing a slot overwrite it: the words only keep the loads).
 *   Timing is the caller's.
 * ------------------------------------------------------------------------ */
int mmv_probe_slots(void);
int mmv_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MATVEC_H */
