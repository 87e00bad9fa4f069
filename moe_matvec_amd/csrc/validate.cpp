// validate.cpp -- host-side argument checks of the C ABI (pure C++).
#include <algorithm>
#include "validate.hpp"

#include "layout.hpp"

namespace mmv {
namespace {

constexpr int64_t kMaxLd = int64_t(1) << 40;
constexpr int64_t kMaxStride = int64_t(1) << 40;  // expert strides (bytes or elements)

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range rng(const void *p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}
Range none() { return Range{0, 0}; }
bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}
bool aligned(const void *p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }
// bytes spanned by `rows` rows of `cols` elements with leading dimension ld
size_t span(int64_t rows, int64_t ld, int64_t cols, size_t elem) {
  return (size_t)(((rows - 1) * ld + cols) * (int64_t)elem);
}
bool bad_batch(int32_t B) { return B < 1 || B > MMV_MAX_BATCH; }
bool bad_moe_batch(int32_t B) { return B < 1 || B > MMV_MOE_MAX_BATCH; }

template <int NO, int NI>
bool any_overlap(const Range (&outs)[NO], const Range (&ins)[NI]) {
  for (int i = 0; i < NO; ++i) {
    for (int j = 0; j < NI; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < NO; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

Range q4_qs(const uint8_t *qs, int64_t N, int64_t K) { return rng(qs, (size_t)(N * K / 2)); }
Range q4_d(const uint16_t *d, int64_t N, int64_t K) { return rng(d, (size_t)(N * K / 32 * 2)); }

}  // namespace

int check_gemv_bf16(const uint16_t *W, int32_t N, int32_t K, int64_t ldw, const float *X,
                    int64_t ldx, int32_t B, const float *Y, int64_t ldy) {
  if (!W || !X || !Y) return MMV_E_NULL;
  if (bad_batch(B)) return MMV_E_BATCH;
  if (N < 1 || K < 8 || K % 8 != 0 || ldw < K || ldx < K || ldy < N) return MMV_E_SHAPE;
  if (ldw > kMaxLd || ldx > kMaxLd || ldy > kMaxLd) return MMV_E_SHAPE;
  if (!aligned(W, 16) || ldw % 8 != 0 || !aligned(X, 16) || ldx % 4 != 0 || !aligned(Y, 4))
    return MMV_E_ALIGN;
  const Range outs[1] = {rng(Y, span(B, ldy, N, 4))};
  const Range ins[2] = {rng(W, span(N, ldw, K, 2)), rng(X, span(B, ldx, K, 4))};
  if (any_overlap(outs, ins)) return MMV_E_ALIAS;
  return MMV_OK;
}

int check_quantize_q8_1(const float *X, int32_t K, int64_t ldx, int32_t B, const void *Xq) {
  if (!X || !Xq) return MMV_E_NULL;
  if (bad_batch(B)) return MMV_E_BATCH;
  if (K < 32 || K % 32 != 0 || ldx < K || ldx > kMaxLd) return MMV_E_SHAPE;
  if (!aligned(X, 16) || ldx % 4 != 0 || !aligned(Xq, 16)) return MMV_E_ALIGN;
  const Range outs[1] = {rng(Xq, q8_1_bytes(K, B))};
  const Range ins[1] = {rng(X, span(B, ldx, K, 4))};
  if (any_overlap(outs, ins)) return MMV_E_ALIAS;
  return MMV_OK;
}

int check_gemv_q4_0(const mmv_q4_0 *W, const float *X, int64_t ldx, const void *Xq,
                    int32_t B, const float *Y, int64_t ldy) {
  if (!W || !W->qs || !W->d || !Y) return MMV_E_NULL;
  if (!X && !Xq) return MMV_E_NULL;
  if (bad_batch(B)) return MMV_E_BATCH;
  const int32_t N = W->N, K = W->K;
  if (N < 1 || K < 32 || K % 32 != 0 || ldy < N || ldy > kMaxLd) return MMV_E_SHAPE;
  if (X && (ldx < K || ldx > kMaxLd)) return MMV_E_SHAPE;
  if ((int64_t)B * K > MMV_Q4_MAX_XK) return MMV_E_SHAPE;
  if (!aligned(W->qs, 16) || !aligned(W->d, 2) || !aligned(Y, 4)) return MMV_E_ALIGN;
  if (X && (!aligned(X, 16) || ldx % 4 != 0)) return MMV_E_ALIGN;
  if (Xq && !aligned(Xq, 16)) return MMV_E_ALIGN;
  const Range y = rng(Y, span(B, ldy, N, 4));
  const Range xq = rng(Xq, q8_1_bytes(K, B));
  const Range w[2] = {q4_qs(W->qs, N, K), q4_d(W->d, N, K)};
  if (X && Xq) {  // Xq is an output here
    const Range outs[2] = {y, xq};
    const Range ins[3] = {w[0], w[1], rng(X, span(B, ldx, K, 4))};
    if (any_overlap(outs, ins)) return MMV_E_ALIAS;
    return MMV_OK;
  }
  const Range outs[1] = {y};
  const Range ins[3] = {w[0], w[1], X ? rng(X, span(B, ldx, K, 4)) : xq};
  if (any_overlap(outs, ins)) return MMV_E_ALIAS;
  return MMV_OK;
}

int check_gemv_q4_0_f32(const mmv_q4_0 *W, const float *X, int64_t ldx, int32_t B,
                        const float *Y, int64_t ldy) {
  if (!W || !W->qs || !W->d || !X || !Y) return MMV_E_NULL;
  if (bad_batch(B)) return MMV_E_BATCH;
  const int32_t N = W->N, K = W->K;
  if (N < 1 || K < 32 || K % 32 != 0 || ldx < K || ldy < N || ldx > kMaxLd || ldy > kMaxLd)
    return MMV_E_SHAPE;
  if ((int64_t)B * K > MMV_Q4F32_MAX_XK) return MMV_E_SHAPE;
  if (!aligned(W->qs, 16) || !aligned(W->d, 2) || !aligned(Y, 4)) return MMV_E_ALIGN;
  if (!aligned(X, 16) || ldx % 4 != 0) return MMV_E_ALIGN;
  const Range outs[1] = {rng(Y, span(B, ldy, N, 4))};
  const Range ins[3] = {q4_qs(W->qs, N, K), q4_d(W->d, N, K), rng(X, span(B, ldx, K, 4))};
  if (any_overlap(outs, ins)) return MMV_E_ALIAS;
  return MMV_OK;
}

size_t argmax_ws_bytes(int32_t N, int32_t B) {
  if (N < 1 || B < 1) return 0;
  return (size_t)B * (size_t)((N + 4095) / 4096) * 8;
}

int check_argmax(const float *Y, int64_t ldy, int32_t N, int32_t B, const int32_t *ids,
                 const float *vals, const void *ws, size_t ws_bytes) {
  if (!Y || !ids || !ws) return MMV_E_NULL;
  if (bad_batch(B)) return MMV_E_BATCH;
  if (N < 1 || ldy < N || ldy > kMaxLd) return MMV_E_SHAPE;
  if (!aligned(Y, 4) || !aligned(ids, 4) || !aligned(vals, 4) || !aligned(ws, 8))
    return MMV_E_ALIGN;
  const size_t need = argmax_ws_bytes(N, B);
  if (ws_bytes < need) return MMV_E_WORKSPACE;
  const Range outs[3] = {rng(ids, 4 * (size_t)B), vals ? rng(vals, 4 * (size_t)B) : none(),
                         rng(ws, need)};
  const Range ins[1] = {rng(Y, span(B, ldy, N, 4))};
  if (any_overlap(outs, ins)) return MMV_E_ALIAS;
  return MMV_OK;
}

int check_route(const float *router, int32_t E, int32_t H, const float *X, int64_t ldx,
                int32_t B, int32_t k, const float *shg, const float *logits,
                const int32_t *ids, const float *weights, const float *shared_w) {
  if (!X || !ids || !weights) return MMV_E_NULL;
  if (router && !logits) return MMV_E_NULL;
  if (bad_moe_batch(B)) return MMV_E_BATCH;
  if (E < 1 || E > MMV_MAX_EXPERTS) return MMV_E_SHAPE;
  if (k < 1 || k > E || k > MMV_MAX_TOPK) return MMV_E_TOPK;
  if (!router && shg) return MMV_E_ARG;
  const int32_t xcols = router ? H : E;
  if (router && (H < 4 || H % 4 != 0)) return MMV_E_SHAPE;
  if (ldx < xcols || ldx > kMaxLd) return MMV_E_SHAPE;
  if (router) {
    if (!aligned(router, 16) || !aligned(X, 16) || ldx % 4 != 0 || !aligned(logits, 4))
      return MMV_E_ALIGN;
    if (shg && !aligned(shg, 16)) return MMV_E_ALIGN;
  } else if (!aligned(X, 4)) {
    return MMV_E_ALIGN;
  }
  if (!aligned(ids, 4) || !aligned(weights, 4) || !aligned(shared_w, 4)) return MMV_E_ALIGN;
  const Range outs[4] = {router ? rng(logits, (size_t)4 * B * (E + 1)) : none(),
                         rng(ids, (size_t)4 * B * k), rng(weights, (size_t)4 * B * k),
                         shared_w ? rng(shared_w, (size_t)4 * B) : none()};
  const Range ins[3] = {router ? rng(router, (size_t)4 * E * H) : none(),
                        rng(X, span(B, ldx, xcols, 4)),
                        shg ? rng(shg, (size_t)4 * H) : none()};
  if (any_overlap(outs, ins)) return MMV_E_ALIAS;
  return MMV_OK;
}

int check_moe_layer(const mmv_moe_layer *L) {
  if (!L) return MMV_E_NULL;
  const int32_t E = L->n_experts, H = L->hidden, I = L->inter, k = L->top_k;
  if (E < 1 || E > MMV_MAX_EXPERTS) return MMV_E_SHAPE;
  if (k < 1 || k > E || k > MMV_MAX_TOPK) return MMV_E_TOPK;
  if (H < 32 || H % 32 != 0 || I < 32 || I % 32 != 0) return MMV_E_SHAPE;
  if (!L->router || !L->gate_qs || !L->up_qs || !L->down_qs || !L->gate_d || !L->up_d ||
      !L->down_d)
    return MMV_E_NULL;
  const int nsh = (L->sh_gate_qs != nullptr) + (L->sh_up_qs != nullptr) +
                  (L->sh_down_qs != nullptr) + (L->sh_gate_d != nullptr) +
                  (L->sh_up_d != nullptr) + (L->sh_down_d != nullptr);
  if (nsh != 0 && nsh != 6) return MMV_E_ARG;
  if (!aligned(L->router, 16) || !aligned(L->gate_qs, 16) || !aligned(L->up_qs, 16) ||
      !aligned(L->down_qs, 16) || !aligned(L->gate_d, 2) || !aligned(L->up_d, 2) ||
      !aligned(L->down_d, 2))
    return MMV_E_ALIGN;
  if (nsh && (!aligned(L->sh_gate_qs, 16) || !aligned(L->sh_up_qs, 16) ||
              !aligned(L->sh_down_qs, 16) || !aligned(L->sh_gate_d, 2) ||
              !aligned(L->sh_up_d, 2) || !aligned(L->sh_down_d, 2)))
    return MMV_E_ALIGN;
  if (L->shared_gate_row && !aligned(L->shared_gate_row, 16)) return MMV_E_ALIGN;
  // expert strides: 0 (contiguous) or at least one expert's plane
  const int64_t nb = (int64_t)I * (H / 32);
  const int64_t qs_st[3] = {L->gate_qs_stride, L->up_qs_stride, L->down_qs_stride};
  const int64_t d_st[3] = {L->gate_d_stride, L->up_d_stride, L->down_d_stride};
  for (int m = 0; m < 3; ++m) {
    if (qs_st[m] != 0 && (qs_st[m] < 16 * nb || qs_st[m] % 16 != 0 || qs_st[m] > kMaxStride))
      return MMV_E_SHAPE;
    if (d_st[m] != 0 && (d_st[m] < nb || d_st[m] > kMaxStride)) return MMV_E_SHAPE;
  }
  return MMV_OK;
}

size_t moe_ws_bytes(const mmv_moe_layer *L, int32_t B) {
  if (check_moe_layer(L) != MMV_OK || bad_moe_batch(B)) return 0;
  return moe_ws_layout(L->n_experts, L->hidden, L->inter, L->top_k, B,
                       L->sh_gate_qs != nullptr).total;
}

namespace {
// ranges of every weight plane of a layer (inputs)
struct LayerRanges {
  Range r[13];
};
// bytes from the first expert's plane to the end of the last one's
size_t stack_bytes(int64_t E, int64_t stride, int64_t one) {
  return (size_t)((stride ? stride : one) * (E - 1) + one);
}
LayerRanges layer_ranges(const mmv_moe_layer *L) {
  const int64_t E = L->n_experts, H = L->hidden, I = L->inter;
  const int64_t nb = I * H / 32;  // blocks of one expert's matrix
  LayerRanges lr;
  lr.r[0] = rng(L->router, (size_t)(4 * E * H));
  lr.r[1] = L->shared_gate_row ? rng(L->shared_gate_row, (size_t)(4 * H)) : none();
  lr.r[2] = rng(L->gate_qs, stack_bytes(E, L->gate_qs_stride, 16 * nb));
  lr.r[3] = rng(L->up_qs, stack_bytes(E, L->up_qs_stride, 16 * nb));
  lr.r[4] = rng(L->down_qs, stack_bytes(E, L->down_qs_stride, 16 * nb));
  lr.r[5] = rng(L->gate_d, 2 * stack_bytes(E, L->gate_d_stride, nb));
  lr.r[6] = rng(L->up_d, 2 * stack_bytes(E, L->up_d_stride, nb));
  lr.r[7] = rng(L->down_d, 2 * stack_bytes(E, L->down_d_stride, nb));
  const bool sh = L->sh_gate_qs != nullptr;
  lr.r[8] = sh ? q4_qs(L->sh_gate_qs, I, H) : none();
  lr.r[9] = sh ? q4_qs(L->sh_up_qs, I, H) : none();
  lr.r[10] = sh ? q4_qs(L->sh_down_qs, H, I) : none();
  lr.r[11] = sh ? q4_d(L->sh_gate_d, I, H) : none();
  lr.r[12] = sh ? q4_d(L->sh_up_d, I, H) : none();
  // sh_down_d is checked separately below (13 slots suffice for the others)
  return lr;
}
bool hits_layer(Range out, const mmv_moe_layer *L) {
  const LayerRanges lr = layer_ranges(L);
  for (const Range &r : lr.r)
    if (overlap(out, r)) return true;
  if (L->sh_down_d && overlap(out, q4_d(L->sh_down_d, L->hidden, L->inter))) return true;
  return false;
}
}  // namespace

int check_mul_mat_id(const mmv_moe_layer *L, const float *X, int64_t ldx, int32_t B,
                     const int32_t *ids, const float *weights, const float *shared_w,
                     const float *Y, int64_t ldy, const void *ws, size_t ws_bytes) {
  const int st = check_moe_layer(L);
  if (st != MMV_OK) return st;
  if (!X || !ids || !weights || !Y) return MMV_E_NULL;
  if (bad_moe_batch(B)) return MMV_E_BATCH;
  const int32_t H = L->hidden, k = L->top_k;
  if (ldx < H || ldy < H || ldx > kMaxLd || ldy > kMaxLd) return MMV_E_SHAPE;
  // x of at most 8 rows is staged per gate/up workgroup (the down projection
  // stages Q8_1(h) on chip only where it fits, else it runs by expert)
  if ((int64_t)std::min<int32_t>(B, MMV_MAX_BATCH) * H > MMV_Q4_MAX_XK) return MMV_E_SHAPE;
  if (!aligned(X, 16) || ldx % 4 != 0 || !aligned(ids, 4) || !aligned(weights, 4) ||
      !aligned(shared_w, 4) || !aligned(Y, 4))
    return MMV_E_ALIGN;
  if (!ws || ws_bytes < moe_ws_bytes(L, B)) return MMV_E_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return MMV_E_ALIGN;
  const Range outs[2] = {rng(Y, span(B, ldy, H, 4)), rng(ws, ws_bytes)};
  const Range ins[4] = {rng(X, span(B, ldx, H, 4)), rng(ids, (size_t)4 * B * k),
                        rng(weights, (size_t)4 * B * k),
                        shared_w ? rng(shared_w, (size_t)4 * B) : none()};
  if (any_overlap(outs, ins)) return MMV_E_ALIAS;
  if (hits_layer(outs[0], L) || hits_layer(outs[1], L)) return MMV_E_ALIAS;
  return MMV_OK;
}

int check_layer_decode(const mmv_moe_layer *L, const float *X, int64_t ldx, int32_t B,
                       const float *Y, int64_t ldy, const int32_t *ids, const float *weights,
                       const void *ws, size_t ws_bytes) {
  const int st = check_moe_layer(L);
  if (st != MMV_OK) return st;
  if (!X || !Y) return MMV_E_NULL;
  if (bad_moe_batch(B)) return MMV_E_BATCH;
  const int32_t H = L->hidden, k = L->top_k;
  if (ldx < H || ldy < H || ldx > kMaxLd || ldy > kMaxLd) return MMV_E_SHAPE;
  // x of at most 8 rows is staged per gate/up workgroup (the down projection
  // stages Q8_1(h) on chip only where it fits, else it runs by expert)
  if ((int64_t)std::min<int32_t>(B, MMV_MAX_BATCH) * H > MMV_Q4_MAX_XK) return MMV_E_SHAPE;
  if (!aligned(X, 16) || ldx % 4 != 0 || !aligned(ids, 4) || !aligned(weights, 4) ||
      !aligned(Y, 4))
    return MMV_E_ALIGN;
  if (!ws || ws_bytes < moe_ws_bytes(L, B)) return MMV_E_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return MMV_E_ALIGN;
  const Range outs[4] = {rng(Y, span(B, ldy, H, 4)), rng(ws, ws_bytes),
                         ids ? rng(ids, (size_t)4 * B * k) : none(),
                         weights ? rng(weights, (size_t)4 * B * k) : none()};
  const Range ins[1] = {rng(X, span(B, ldx, H, 4))};
  if (any_overlap(outs, ins)) return MMV_E_ALIAS;
  for (const Range &o : outs)
    if (hits_layer(o, L)) return MMV_E_ALIAS;
  return MMV_OK;
}

}  // namespace mmv
