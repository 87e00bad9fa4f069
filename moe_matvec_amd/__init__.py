"""Python binding of libmoe_matvec.so (include/moe_matvec.h).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch tensors on a ROCm device; calls enqueue on the current
torch stream (or the one given) and return without synchronizing.

The library must have been built in-tree (``python -m moe_matvec_amd.build``);
if it is missing, importing the binding raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "MatvecError", "Q4_0", "MoeLayer", "library_path", "lib",
    "gemv_bf16", "quantize_q8_1", "q8_1_bytes", "gemv_q4_0", "gemv_q4_0_f32",
    "argmax_rows", "argmax_workspace_bytes", "Q4F32_MAX_XK",
    "moe_route_topk", "moe_mul_mat_id", "moe_layer_decode", "moe_workspace_bytes",
    "MAX_BATCH", "MOE_MAX_BATCH", "MAX_EXPERTS", "MAX_TOPK", "Q4_MAX_XK", "stream_read", "split_q8_1",
    "PATH", "set_path", "get_path", "moe_layer_decode_noalloc", "NOALLOC_WS_BYTES",
]

MAX_BATCH = 8
MOE_MAX_BATCH = 64  # MoE calls: verify / prefill batches
MAX_EXPERTS = 1024
MAX_TOPK = 16
Q4_MAX_XK = 49152
Q4F32_MAX_XK = 36864
NOALLOC_WS_BYTES = 8 << 20  # the library's own workspace of moe_layer_decode_noalloc

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmoe_matvec.so")


class MatvecError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().mmv_status_str(status).decode()
        if status == -8:
            msg += f" (hipError {lib().mmv_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [status {status}]")


_P = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64


class _Q4(C.Structure):
    _fields_ = [("qs", _P), ("d", _P), ("N", _i32), ("K", _i32)]


class _Layer(C.Structure):
    _fields_ = [("n_experts", _i32), ("hidden", _i32), ("inter", _i32), ("top_k", _i32),
                ("router", _P), ("shared_gate_row", _P),
                ("gate_qs", _P), ("up_qs", _P), ("down_qs", _P),
                ("gate_d", _P), ("up_d", _P), ("down_d", _P),
                ("sh_gate_qs", _P), ("sh_up_qs", _P), ("sh_down_qs", _P),
                ("sh_gate_d", _P), ("sh_up_d", _P), ("sh_down_d", _P),
                ("gate_qs_stride", C.c_int64), ("up_qs_stride", C.c_int64),
                ("down_qs_stride", C.c_int64), ("gate_d_stride", C.c_int64),
                ("up_d_stride", C.c_int64), ("down_d_stride", C.c_int64)]


class _Debug(C.Structure):
    _fields_ = [("h", _P), ("unique", _P), ("offsets", _P), ("pairs", _P), ("n_unique", _P),
                ("x_q8", _P), ("gate_out", _P), ("up_out", _P), ("h_q8", _P), ("down_out", _P)]


_DEBUG_FIELDS = [f for f, _ in _Debug._fields_]

# kernel-variant switches of include/moe_matvec_testing.h (tests and measurements only)
PATH = dict(BF16_ROWS=0, BF16_WAVES=1, BF16_XL=2, BF16_ML=3, Q4_RP=4, Q4_GENERIC=5,
            Q4_WG_PER_CU=6, MOE_TOPK=7, MOE_DOWN=8, Q4F32_MF=9, Q4_MF=10)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is not built; run `python -m moe_matvec_amd.build`")
        L = C.CDLL(library_path)
        sig = {
            "mmv_status_str": (C.c_char_p, [C.c_int]),
            "mmv_last_hip_error": (C.c_int, []),
            "mmv_q8_1_bytes": (C.c_size_t, [_i32, _i32]),
            "gemv_bf16": (C.c_int, [_P, _i32, _i32, _i64, _P, _i64, _i32, _P, _i64, _P]),
            "quantize_q8_1": (C.c_int, [_P, _i32, _i64, _i32, _P, _P]),
            "gemv_q4_0": (C.c_int, [C.POINTER(_Q4), _P, _i64, _P, _i32, _P, _i64, _P]),
            "gemv_q4_0_f32": (C.c_int, [C.POINTER(_Q4), _P, _i64, _i32, _P, _i64, _P]),
            "mmv_argmax_workspace_bytes": (C.c_size_t, [_i32, _i32]),
            "argmax_rows": (C.c_int, [_P, _i64, _i32, _i32, _P, _P, _P, C.c_size_t, _P]),
            "moe_route_topk": (C.c_int, [_P, _i32, _i32, _P, _i64, _i32, _i32, _P, _P, _P,
                                         _P, _P, _P]),
            "moe_workspace_bytes": (C.c_size_t, [C.POINTER(_Layer), _i32]),
            "moe_mul_mat_id": (C.c_int, [C.POINTER(_Layer), _P, _i64, _i32, _P, _P, _P, _P,
                                         _i64, _P, C.c_size_t, C.POINTER(_Debug), _P]),
            "moe_layer_decode": (C.c_int, [C.POINTER(_Layer), _P, _i64, _i32, _P, _i64, _P,
                                           _P, _P, C.c_size_t, _P]),
            "mmv_noalloc_ws_bytes": (C.c_size_t, []),
            "moe_layer_decode_noalloc": (C.c_int, [C.POINTER(_Layer), _P, _i64, _i32, _P, _i64,
                                                   _P, _P, _P]),
            "mmv_timeline": (C.c_size_t, [_P, C.c_int, _P]),
            "mmv_set_path": (C.c_int, [C.c_int, C.c_int]),
            "mmv_get_path": (C.c_int, [C.c_int]),
            "mmv_probe_slots": (C.c_int, []),
            "mmv_stream_read": (C.c_int, [_P, C.c_size_t, _P, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def set_path(name: str, value: int) -> int:
    """Force a kernel variant (include/moe_matvec_testing.h; tests and
    measurements only); 0 restores the automatic choice.  Returns the previous
    value."""
    return int(lib().mmv_set_path(PATH[name], int(value)))


def get_path(name: str) -> int:
    return int(lib().mmv_get_path(PATH[name]))


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn, status):
    if status != 0:
        raise MatvecError(fn, status)


def _ld(x2):
    """Leading dimension of a [B, K] view (any value >= K is valid for B = 1)."""
    return x2.stride(0) if x2.shape[0] > 1 else x2.shape[1]


class Q4_0:
    """Planar Q4_0 matrix: qs uint8 [N, K/32, 16] (split-nibble), d float16 [N, K/32]."""

    def __init__(self, qs: torch.Tensor, d: torch.Tensor):
        if qs.dtype != torch.uint8 or d.dtype != torch.float16:
            raise TypeError("Q4_0 needs qs uint8 and d float16")
        if qs.dim() != 3 or qs.shape[2] != 16 or d.shape != qs.shape[:2]:
            raise ValueError("Q4_0 shapes: qs [N, K/32, 16], d [N, K/32]")
        if not (qs.is_contiguous() and d.is_contiguous()):
            raise ValueError("Q4_0 planes must be contiguous")
        self.qs, self.d = qs, d
        self.N, self.K = qs.shape[0], qs.shape[1] * 32
        self._s = _Q4(qs.data_ptr(), d.data_ptr(), self.N, self.K)

    @property
    def nbytes(self):
        return self.qs.numel() + 2 * self.d.numel()


# ---------------------------------------------------------------------------
# dense / quantized GEMV
# ---------------------------------------------------------------------------

def gemv_bf16(W: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """y[b, n] = sum_k W[n, k] x[b, k]; W bf16 [N, K], x fp32 [K] or [B, K] -> fp32."""
    if W.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("W must be bfloat16 (or its 16-bit pattern)")
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be [N, K] with unit inner stride")
    x2, squeeze = (x.unsqueeze(0), True) if x.dim() == 1 else (x, False)
    if x2.dtype != torch.float32 or x2.stride(-1) != 1:
        raise TypeError("x must be float32 with unit inner stride")
    N, K = W.shape
    B = x2.shape[0]
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=W.device)
    y2 = out.unsqueeze(0) if out.dim() == 1 else out
    _check("gemv_bf16", lib().gemv_bf16(W.data_ptr(), N, K, W.stride(0), x2.data_ptr(),
                                        _ld(x2), B, y2.data_ptr(), _ld(y2), _stream(stream)))
    return out[0] if (squeeze and out.dim() == 2) else out


def q8_1_bytes(K: int, B: int) -> int:
    return int(lib().mmv_q8_1_bytes(K, B))


def quantize_q8_1(x: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """Planar Q8_1 of fp32 x [B, K]: returns a uint8 buffer of q8_1_bytes(K, B)."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    if x2.dtype != torch.float32 or x2.stride(-1) != 1:
        raise TypeError("x must be float32 with unit inner stride")
    B, K = x2.shape
    nbytes = q8_1_bytes(K, B)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check("quantize_q8_1", lib().quantize_q8_1(x2.data_ptr(), K, _ld(x2), B,
                                                out.data_ptr(), _stream(stream)))
    return out


def split_q8_1(buf: torch.Tensor, B: int, K: int):
    """Views of a planar Q8_1 buffer: (codes int8 [B, K], ds uint16-bits int16 [B, K/32, 2])."""
    codes = buf[:B * K].view(torch.int8).view(B, K)
    ds = buf[B * K:B * K + 4 * B * (K // 32)].view(torch.int16).view(B, K // 32, 2)
    return codes, ds


def gemv_q4_0(W: Q4_0, x: torch.Tensor | None = None, xq: torch.Tensor | None = None,
              B: int | None = None, out: torch.Tensor | None = None, stream=None):
    """y = W (x) Q8_1(x).  Pass fp32 x [B, K] (quantized inside the product),
    or a planar Q8_1 buffer xq with its row count B, or both: then x is
    quantized into xq (uint8, q8_1_bytes(K, B) bytes, overwritten) by a
    separate pass and the product reads xq."""
    if x is None and xq is None:
        raise ValueError("give x, xq or both")
    if x is not None:
        x2 = x.unsqueeze(0) if x.dim() == 1 else x
        if x2.dtype != torch.float32 or x2.stride(-1) != 1:
            raise TypeError("x must be float32 with unit inner stride")
        B = x2.shape[0]
        xp, ldx = x2.data_ptr(), _ld(x2)
        dev = x.device
    else:
        if B is None:
            raise ValueError("B is required with xq")
        xp, ldx, dev = None, W.K, xq.device
    if xq is not None and (xq.dtype != torch.uint8 or xq.numel() < q8_1_bytes(W.K, B)):
        raise ValueError("xq must be uint8 with at least q8_1_bytes(K, B) bytes")
    if out is None:
        out = torch.empty((B, W.N), dtype=torch.float32, device=dev)
    y2 = out.unsqueeze(0) if out.dim() == 1 else out
    _check("gemv_q4_0", lib().gemv_q4_0(C.byref(W._s), xp, ldx, _ptr(xq), B,
                                        y2.data_ptr(), _ld(y2), _stream(stream)))
    return out


def gemv_q4_0_f32(W: Q4_0, x: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """W4A16: y = W x with Q4_0 weights and fp32 activations (no Q8_1 step);
    x fp32 [B, K] or [K]."""
    x2, squeeze = (x.unsqueeze(0), True) if x.dim() == 1 else (x, False)
    if x2.dtype != torch.float32 or x2.stride(-1) != 1:
        raise TypeError("x must be float32 with unit inner stride")
    B = x2.shape[0]
    if out is None:
        out = torch.empty((B, W.N), dtype=torch.float32, device=x.device)
    y2 = out.unsqueeze(0) if out.dim() == 1 else out
    _check("gemv_q4_0_f32", lib().gemv_q4_0_f32(C.byref(W._s), x2.data_ptr(), _ld(x2), B,
                                                y2.data_ptr(), _ld(y2), _stream(stream)))
    return out[0] if (squeeze and out.dim() == 2) else out


def argmax_workspace_bytes(N: int, B: int) -> int:
    return int(lib().mmv_argmax_workspace_bytes(N, B))


def argmax_rows(y: torch.Tensor, ids: torch.Tensor | None = None, vals: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None):
    """Per row of fp32 y [B, N]: index (int32 [B]) of the largest value, lowest
    index on ties; returns (ids, vals)."""
    y2 = y.unsqueeze(0) if y.dim() == 1 else y
    if y2.dtype != torch.float32 or y2.stride(-1) != 1:
        raise TypeError("y must be float32 with unit inner stride")
    B, N = y2.shape
    if ids is None:
        ids = torch.empty(B, dtype=torch.int32, device=y.device)
    if vals is None:
        vals = torch.empty(B, dtype=torch.float32, device=y.device)
    if workspace is None:
        workspace = torch.empty(argmax_workspace_bytes(N, B), dtype=torch.uint8, device=y.device)
    _check("argmax_rows", lib().argmax_rows(y2.data_ptr(), _ld(y2), N, B, ids.data_ptr(),
                                            _ptr(vals), workspace.data_ptr(), workspace.numel(),
                                            _stream(stream)))
    return ids, vals


# ---------------------------------------------------------------------------
# MoE
# ---------------------------------------------------------------------------

def moe_route_topk(router: torch.Tensor | None, x: torch.Tensor, k: int,
                   shared_gate_row: torch.Tensor | None = None, n_experts: int | None = None,
                   logits=None, ids=None, weights=None, shared_w=None, stream=None):
    """Router logits, top-k ids (descending, lower index on ties) and renormalised
    weights.  With router=None, x holds [B, E] logits.  Returns (ids, weights,
    shared_w, logits)."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    if x2.dtype != torch.float32 or x2.stride(-1) != 1:
        raise TypeError("x must be float32 with unit inner stride")
    B = x2.shape[0]
    dev = x.device
    if router is not None:
        E, H = router.shape
        if logits is None:
            logits = torch.empty((B, E + 1), dtype=torch.float32, device=dev)
    else:
        E, H = (n_experts or x2.shape[1]), 0
    if ids is None:
        ids = torch.empty((B, k), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((B, k), dtype=torch.float32, device=dev)
    if shared_w is None:
        shared_w = torch.empty((B,), dtype=torch.float32, device=dev)
    _check("moe_route_topk", lib().moe_route_topk(
        _ptr(router), E, H, x2.data_ptr(), _ld(x2), B, k, _ptr(shared_gate_row),
        _ptr(logits), ids.data_ptr(), weights.data_ptr(), shared_w.data_ptr(),
        _stream(stream)))
    return ids, weights, shared_w, logits


class MoeLayer:
    """One MoE layer's device tensors (planar Q4_0, experts stacked expert-major).

    gate/up: qs uint8 [E, I, H/32, 16], d float16 [E, I, H/32]
    down:    qs uint8 [E, H, I/32, 16], d float16 [E, H, I/32]
    shared:  dict with the same keys without the E dimension, or None.
    A routed tensor may step between experts by more than one expert's size
    (a view such as big[:, :I] of a padded stack): each expert must be
    contiguous; the expert stride goes to the library.
    """

    def __init__(self, router, gate_qs, gate_d, up_qs, up_d, down_qs, down_d, top_k,
                 shared=None, shared_gate_row=None):
        self.router = router
        self.E, self.H = router.shape
        self.I = gate_qs.shape[1]
        self.k = top_k
        self.t = dict(gate_qs=gate_qs, gate_d=gate_d, up_qs=up_qs, up_d=up_d,
                      down_qs=down_qs, down_d=down_d)
        self.shared = shared
        self.shared_gate_row = shared_gate_row
        s = _Layer()
        s.n_experts, s.hidden, s.inter, s.top_k = self.E, self.H, self.I, top_k
        s.router = router.data_ptr()
        s.shared_gate_row = _ptr(shared_gate_row)
        for name, t in self.t.items():
            if not t[0].is_contiguous():
                raise ValueError(f"{name}: each expert must be contiguous")
            setattr(s, name, t.data_ptr())
            # bytes (qs, uint8) or elements (d, fp16) from one expert to the next
            setattr(s, name + "_stride", t.stride(0) if self.E > 1 else 0)
        if shared is not None:
            for name in ("gate_qs", "gate_d", "up_qs", "up_d", "down_qs", "down_d"):
                setattr(s, "sh_" + name, shared[name].data_ptr())
        self._s = s

    @property
    def has_shared(self):
        return self.shared is not None

    def npairs(self, B):
        return B * self.k + (B if self.has_shared else 0)

    def expert_bytes(self):
        """Bytes of one expert's gate+up+down weights."""
        nb = (self.I * self.H) // 32
        return 3 * (nb * 16 + nb * 2)


def moe_workspace_bytes(layer: MoeLayer, B: int) -> int:
    return int(lib().moe_workspace_bytes(C.byref(layer._s), B))


def moe_mul_mat_id(layer: MoeLayer, x: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor,
                   shared_w: torch.Tensor | None = None, out=None, workspace=None,
                   debug: dict | None = None, stream=None):
    """Routed + shared expert FFN.  debug may hold device tensors that receive
    staged results (P = B*k + B with a shared expert, else B*k): h, gate_out,
    up_out [P, I] f32; down_out [P, H] f32; x_q8 (q8_1_bytes(H, B) bytes) and
    h_q8 (q8_1_bytes(I, P) bytes) planar Q8_1; unique, offsets, pairs,
    n_unique int32."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    B = x2.shape[0]
    if out is None:
        out = torch.empty((B, layer.H), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(moe_workspace_bytes(layer, B), dtype=torch.uint8,
                                device=x.device)
    dbg = None
    if debug is not None:
        unknown = set(debug) - set(_DEBUG_FIELDS)
        if unknown:
            raise ValueError(f"unknown debug fields {sorted(unknown)}")
        dbg = _Debug(*(_ptr(debug.get(n)) for n in _DEBUG_FIELDS))
    y2 = out.unsqueeze(0) if out.dim() == 1 else out
    _check("moe_mul_mat_id", lib().moe_mul_mat_id(
        C.byref(layer._s), x2.data_ptr(), _ld(x2), B, ids.data_ptr(), weights.data_ptr(),
        _ptr(shared_w), y2.data_ptr(), _ld(y2), workspace.data_ptr(), workspace.numel(),
        C.byref(dbg) if dbg is not None else None, _stream(stream)))
    return out


def moe_layer_decode(layer: MoeLayer, x: torch.Tensor, out=None, workspace=None, ids=None,
                     weights=None, stream=None):
    """Whole MoE layer (route + experts) on device; returns out [B, H]."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    B = x2.shape[0]
    if out is None:
        out = torch.empty((B, layer.H), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(moe_workspace_bytes(layer, B), dtype=torch.uint8,
                                device=x.device)
    y2 = out.unsqueeze(0) if out.dim() == 1 else out
    _check("moe_layer_decode", lib().moe_layer_decode(
        C.byref(layer._s), x2.data_ptr(), _ld(x2), B, y2.data_ptr(), _ld(y2), _ptr(ids),
        _ptr(weights), workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out


def moe_layer_decode_noalloc(layer: MoeLayer, x: torch.Tensor, out=None, ids=None, weights=None,
                             stream=None):
    """moe_layer_decode with the library's own workspace (allocates nothing
    on the device when `out` is given; calls on one GPU must not overlap)."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    B = x2.shape[0]
    if out is None:
        out = torch.empty((B, layer.H), dtype=torch.float32, device=x.device)
    y2 = out.unsqueeze(0) if out.dim() == 1 else out
    _check("moe_layer_decode_noalloc", lib().moe_layer_decode_noalloc(
        C.byref(layer._s), x2.data_ptr(), _ld(x2), B, y2.data_ptr(), _ld(y2), _ptr(ids),
        _ptr(weights), _stream(stream)))
    return out


def stream_read(buf: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """Read-bandwidth probe: streams every byte of buf once (timing is the caller's)."""
    if out is None:
        out = torch.empty(lib().mmv_probe_slots(), dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check("mmv_stream_read", lib().mmv_stream_read(buf.data_ptr(), nbytes - nbytes % 16,
                                                    out.data_ptr(), _stream(stream)))
    return out
