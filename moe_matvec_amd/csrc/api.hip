// api.hip -- the extern "C" entry points of moe_matvec.h: validate on the
// host (validate.cpp, no device access), then enqueue on the caller's
// stream.  No allocation, no synchronization, no host reads of device data.
#include <atomic>
#include <mutex>

#include "../../include/moe_matvec.h"
#include "../../include/moe_matvec_testing.h"
#include "launch.hpp"
#include "layout.hpp"
#include "validate.hpp"

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MMV_OK;
  g_last_hip = (int)e;
  return MMV_E_HIP;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// kernel-variant switches (moe_matvec_testing.h): 0 = automatic
std::atomic<int> g_path[MMV_PATH_COUNT];

}  // namespace

// ---------------------------------------------------------------------------
// The library's own MoE workspace for moe_layer_decode_noalloc: one array per
// GPU, held from the module load until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: the kernels get
// the device address hipGetSymbolAddress returns, fetched once per device
// with that device current, and only that address is used from then on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MMV_NOALLOC_WS_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<uint8_t *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// device address of this device's scratch array (looked up on first use)
hipError_t scratch_on_current_device(uint8_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint8_t *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!addr) return hipErrorInvalidSymbol;
      p = static_cast<uint8_t *>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

namespace mmv {
int path_switch(int which) {
  if (which < 0 || which >= MMV_PATH_COUNT) return 0;
  return g_path[which].load(std::memory_order_relaxed);
}

// a data race between first calls on a device only stores the same value
// twice; a device the query fails on counts as 256 CUs
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace mmv

extern "C" {

const char *mmv_status_str(int status) {
  switch (status) {
    case MMV_OK: return "ok";
    case MMV_E_NULL: return "a required pointer is NULL";
    case MMV_E_SHAPE: return "a size is out of range or not a multiple of the block size";
    case MMV_E_ALIGN: return "a pointer or leading dimension is misaligned";
    case MMV_E_BATCH: return "batch rows outside 1..8 (MoE entry points: 1..64)";
    case MMV_E_TOPK: return "top_k outside 1..min(E, 16)";
    case MMV_E_WORKSPACE: return "workspace missing or too small";
    case MMV_E_ALIAS: return "an output overlaps an input";
    case MMV_E_HIP: return "HIP launch failed";
    case MMV_E_ARG: return "inconsistent arguments";
  }
  return "unknown status";
}

int mmv_last_hip_error(void) { return g_last_hip; }

int mmv_set_path(int which, int value) {
  if (which < 0 || which >= MMV_PATH_COUNT) return MMV_E_ARG;
  return g_path[which].exchange(value, std::memory_order_relaxed);
}

int mmv_get_path(int which) { return mmv::path_switch(which); }

size_t mmv_q8_1_bytes(int32_t K, int32_t B) {
  if (K < 32 || K % 32 != 0 || B < 1) return 0;
  return mmv::q8_1_bytes(K, B);
}

int gemv_bf16(const uint16_t *W, int32_t N, int32_t K, int64_t ldw, const float *X,
              int64_t ldx, int32_t B, float *Y, int64_t ldy, void *stream) {
  const int st = mmv::check_gemv_bf16(W, N, K, ldw, X, ldx, B, Y, ldy);
  if (st != MMV_OK) return st;
  return hip_status(mmv::run_gemv_bf16(W, N, K, ldw, X, ldx, B, Y, ldy, as_stream(stream)));
}

int quantize_q8_1(const float *X, int32_t K, int64_t ldx, int32_t B, void *Xq, void *stream) {
  const int st = mmv::check_quantize_q8_1(X, K, ldx, B, Xq);
  if (st != MMV_OK) return st;
  return hip_status(mmv::run_quantize_q8_1(X, K, ldx, B, static_cast<uint8_t *>(Xq),
                                           as_stream(stream)));
}

int gemv_q4_0(const mmv_q4_0 *W, const float *X, int64_t ldx, const void *Xq, int32_t B,
              float *Y, int64_t ldy, void *stream) {
  const int st = mmv::check_gemv_q4_0(W, X, ldx, Xq, B, Y, ldy);
  if (st != MMV_OK) return st;
  return hip_status(mmv::run_gemv_q4_0(W->qs, W->d, W->N, W->K, X, ldx,
                                       static_cast<const uint8_t *>(Xq), B, Y, ldy,
                                       as_stream(stream)));
}

int gemv_q4_0_f32(const mmv_q4_0 *W, const float *X, int64_t ldx, int32_t B, float *Y,
                  int64_t ldy, void *stream) {
  const int st = mmv::check_gemv_q4_0_f32(W, X, ldx, B, Y, ldy);
  if (st != MMV_OK) return st;
  return hip_status(mmv::run_gemv_q4_0_f32(W->qs, W->d, W->N, W->K, X, ldx, B, Y, ldy,
                                           as_stream(stream)));
}

size_t mmv_argmax_workspace_bytes(int32_t N, int32_t B) { return mmv::argmax_ws_bytes(N, B); }

int argmax_rows(const float *Y, int64_t ldy, int32_t N, int32_t B, int32_t *ids, float *vals,
                void *workspace, size_t ws_bytes, void *stream) {
  const int st = mmv::check_argmax(Y, ldy, N, B, ids, vals, workspace, ws_bytes);
  if (st != MMV_OK) return st;
  return hip_status(mmv::run_argmax(Y, ldy, N, B, ids, vals, static_cast<uint64_t *>(workspace),
                                    as_stream(stream)));
}

int moe_route_topk(const float *router, int32_t E, int32_t H, const float *X, int64_t ldx,
                   int32_t B, int32_t k, const float *shared_gate_row, float *logits,
                   int32_t *ids, float *weights, float *shared_w, void *stream) {
  const int st = mmv::check_route(router, E, H, X, ldx, B, k, shared_gate_row, logits, ids,
                                  weights, shared_w);
  if (st != MMV_OK) return st;
  return hip_status(mmv::run_moe_route(router, E, H, X, ldx, B, k, shared_gate_row, logits,
                                       ids, weights, shared_w, as_stream(stream)));
}

size_t moe_workspace_bytes(const mmv_moe_layer *L, int32_t B) { return mmv::moe_ws_bytes(L, B); }

int moe_mul_mat_id(const mmv_moe_layer *L, const float *X, int64_t ldx, int32_t B,
                   const int32_t *ids, const float *weights, const float *shared_w, float *Y,
                   int64_t ldy, void *workspace, size_t ws_bytes, const mmv_moe_debug *dbg,
                   void *stream) {
  const int st = mmv::check_mul_mat_id(L, X, ldx, B, ids, weights, shared_w, Y, ldy,
                                       workspace, ws_bytes);
  if (st != MMV_OK) return st;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  return hip_status(mmv::run_moe_experts(*L, X, ldx, B, ids, weights, shared_w, Y, ldy, ws,
                                         dbg, as_stream(stream)));
}

int moe_layer_decode(const mmv_moe_layer *L, const float *X, int64_t ldx, int32_t B, float *Y,
                     int64_t ldy, int32_t *ids, float *weights, void *workspace,
                     size_t ws_bytes, void *stream) {
  const int st =
      mmv::check_layer_decode(L, X, ldx, B, Y, ldy, ids, weights, workspace, ws_bytes);
  if (st != MMV_OK) return st;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const mmv::MoeWsLayout lay =
      mmv::moe_ws_layout(L->n_experts, L->hidden, L->inter, L->top_k, B,
                         L->sh_gate_qs != nullptr);
  int32_t *id = ids ? ids : reinterpret_cast<int32_t *>(ws + lay.ids);
  float *w = weights ? weights : reinterpret_cast<float *>(ws + lay.weights);
  return hip_status(mmv::run_moe_layer(*L, X, ldx, B, id, w, Y, ldy, ws, as_stream(stream)));
}

size_t mmv_noalloc_ws_bytes(void) { return MMV_NOALLOC_WS_BYTES; }

int moe_layer_decode_noalloc(const mmv_moe_layer *L, const float *X, int64_t ldx, int32_t B,
                             float *Y, int64_t ldy, int32_t *ids, float *weights,
                             void *stream) {
  // sizes first (no HIP call): a layer or batch whose workspace exceeds the
  // library's array is refused before anything else
  const size_t need = mmv::moe_ws_bytes(L, B);
  if (need > MMV_NOALLOC_WS_BYTES) return MMV_E_WORKSPACE;
  if (need == 0) {  // the layer or B is invalid: report why
    const int st = mmv::check_layer_decode(L, X, ldx, B, Y, ldy, ids, weights, nullptr, 0);
    return st != MMV_OK ? st : MMV_E_SHAPE;
  }
  uint8_t *ws = nullptr;
  const hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return hip_status(e);
  const int st = mmv::check_layer_decode(L, X, ldx, B, Y, ldy, ids, weights, ws,
                                         MMV_NOALLOC_WS_BYTES);
  if (st != MMV_OK) return st;
  const mmv::MoeWsLayout lay =
      mmv::moe_ws_layout(L->n_experts, L->hidden, L->inter, L->top_k, B,
                         L->sh_gate_qs != nullptr);
  int32_t *id = ids ? ids : reinterpret_cast<int32_t *>(ws + lay.ids);
  float *w = weights ? weights : reinterpret_cast<float *>(ws + lay.weights);
  return hip_status(mmv::run_moe_layer(*L, X, ldx, B, id, w, Y, ldy, ws, as_stream(stream)));
}

int mmv_probe_slots(void) { return mmv::probe_slots(); }

int mmv_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream) {
  if (!buf || !out) return MMV_E_NULL;
  // a dispatch counts its work-items in 32 bits: at most 2^24 workgroups of 32 KiB
  if (bytes < 16 || bytes % 16 != 0 || bytes > ((size_t)1 << 38)) return MMV_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 4 != 0)
    return MMV_E_ALIGN;
  const uintptr_t o = reinterpret_cast<uintptr_t>(out), b = reinterpret_cast<uintptr_t>(buf);
  if (o < b + bytes && b < o + 4 * (size_t)mmv::probe_slots()) return MMV_E_ALIAS;
  return hip_status(mmv::run_stream_read(buf, bytes, out, as_stream(stream)));
}

}  // extern "C"
