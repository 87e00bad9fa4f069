"""ctypes wrapper of the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path (moe_matvec_amd).

All arrays are numpy; shapes follow oracle.h.  The shared library is built
in-tree with gcc (``build()``); ``lib()`` builds it only if it is missing.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into oracle/liboracle.so with plain gcc."""
    cmd = ["gcc", *CFLAGS, os.path.join(_HERE, "oracle.c"), "-o", _SO + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_P = C.c_void_p
_I = C.c_int
_L = C.c_long


class _Moe(C.Structure):
    _fields_ = [("E", _I), ("H", _I), ("I", _I), ("k", _I),
                ("router", _P), ("shared_gate_row", _P),
                ("gate_qs", _P), ("up_qs", _P), ("down_qs", _P),
                ("gate_d", _P), ("up_d", _P), ("down_d", _P),
                ("sh_gate_qs", _P), ("sh_up_qs", _P), ("sh_down_qs", _P),
                ("sh_gate_d", _P), ("sh_up_d", _P), ("sh_down_d", _P)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = C.CDLL(_SO)
        sig = {
            "orc_f32_to_f16": (C.c_uint16, [C.c_float]),
            "orc_f16_to_f32": (C.c_float, [C.c_uint16]),
            "orc_f32_to_bf16": (C.c_uint16, [C.c_float]),
            "orc_bf16_to_f32": (C.c_float, [C.c_uint16]),
            "orc_f32_to_f16_n": (None, [_P, _P, _L]),
            "orc_f16_to_f32_n": (None, [_P, _P, _L]),
            "orc_f32_to_bf16_n": (None, [_P, _P, _L]),
            "orc_bf16_to_f32_n": (None, [_P, _P, _L]),
            "orc_gemv_bf16": (None, [_P, _I, _I, _L, _P, _L, _I, _P]),
            "orc_quantize_q8_1": (None, [_P, _I, _L, _I, _P, _P]),
            "orc_q4_0_block_sums": (None, [_P, _I, _I, _P, _I, _P]),
            "orc_gemv_q4_0": (None, [_P, _P, _I, _I, _P, _P, _I, _P]),
            "orc_gemv_q4_0_f32": (None, [_P, _P, _I, _I, _P, _L, _I, _P]),
            "orc_argmax": (None, [_P, _L, _I, _I, _P]),
            "orc_router_logits": (None, [_P, _I, _I, _P, _L, _I, _P]),
            "orc_topk": (None, [_P, _I, _L, _I, _I, _P]),
            "orc_gate_weights": (None, [_P, _L, _P, _I, _I, _P]),
            "orc_gather": (_I, [_P, _I, _I, _P, _P, _P]),
            "orc_moe_route": (None, [C.POINTER(_Moe), _P, _L, _I, _P, _P, _P, _P]),
            "orc_moe_gate_up": (None, [C.POINTER(_Moe), _P, _L, _I, _P, _P]),
            "orc_moe_down": (None, [C.POINTER(_Moe), _P, _P, _I, _P, _P, _P, _P]),
            "orc_moe_layer": (None, [C.POINTER(_Moe), _P, _L, _I, _P, _P, _P, _P, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


# ---- number formats --------------------------------------------------------

def f32_to_f16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_n(_p(x), _p(out), x.size)
    return out


def f16_to_f32(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_n(_p(h), _p(out), h.size)
    return out


def f32_to_bf16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_n(_p(x), _p(out), x.size)
    return out


def bf16_to_f32(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_bf16_to_f32_n(_p(h), _p(out), h.size)
    return out


# ---- GEMV ------------------------------------------------------------------

def gemv_bf16(W, X, K=None):
    """W: uint16 [N, ldw] (bf16 bits), X: float32 [B, ldx]; returns float64 [B, N]."""
    W = _c(W, np.uint16)
    X = _c(np.atleast_2d(X), np.float32)
    N, ldw = W.shape
    B, ldx = X.shape
    K = ldw if K is None else K
    assert K <= ldw and K <= ldx
    Y = np.empty((B, N), np.float64)
    lib().orc_gemv_bf16(_p(W), N, K, ldw, _p(X), ldx, B, _p(Y))
    return Y


def quantize_q8_1(X, K=None):
    """X: float32 [B, ldx]; returns (q int8 [B, K], ds uint16 [B, K/32, 2])."""
    X = _c(np.atleast_2d(X), np.float32)
    B, ldx = X.shape
    K = ldx if K is None else K
    assert K % 32 == 0
    q = np.empty((B, K), np.int8)
    ds = np.empty((B, K // 32, 2), np.uint16)
    lib().orc_quantize_q8_1(_p(X), K, ldx, B, _p(q), _p(ds))
    return q, ds


def q4_0_block_sums(qs, xq):
    """qs: uint8 [N, K/32, 16]; xq: int8 [B, K]; returns int32 [B, N, K/32]."""
    qs = _c(qs, np.uint8)
    xq = _c(np.atleast_2d(xq), np.int8)
    N, nb, _ = qs.shape
    B, K = xq.shape
    assert K == nb * 32
    out = np.empty((B, N, nb), np.int32)
    lib().orc_q4_0_block_sums(_p(qs), N, K, _p(xq), B, _p(out))
    return out


def gemv_q4_0(qs, dw, xq, xds):
    """qs uint8 [N, nb, 16], dw uint16 [N, nb], xq int8 [B, K], xds uint16 [B, nb, 2]."""
    qs = _c(qs, np.uint8)
    dw = _c(dw, np.uint16)
    xq = _c(np.atleast_2d(xq), np.int8)
    xds = _c(xds, np.uint16).reshape(xq.shape[0], -1, 2)
    N, nb, _ = qs.shape
    B, K = xq.shape
    assert K == nb * 32 and dw.shape == (N, nb) and xds.shape[1] == nb
    Y = np.empty((B, N), np.float64)
    lib().orc_gemv_q4_0(_p(qs), _p(dw), N, K, _p(xq), _p(xds), B, _p(Y))
    return Y


def gemv_q4_0_f32(qs, dw, X):
    """W4A16: qs uint8 [N, nb, 16], dw uint16 [N, nb], X float32 [B, K] -> float64 [B, N]."""
    qs = _c(qs, np.uint8)
    dw = _c(dw, np.uint16)
    X = _c(np.atleast_2d(X), np.float32)
    N, nb, _ = qs.shape
    B, K = X.shape
    assert K == nb * 32 and dw.shape == (N, nb)
    Y = np.empty((B, N), np.float64)
    lib().orc_gemv_q4_0_f32(_p(qs), _p(dw), N, K, _p(X), K, B, _p(Y))
    return Y


def argmax(Y):
    """Y float32 [B, N] -> int32 [B]: largest value, lowest index on ties."""
    Y = _c(np.atleast_2d(Y), np.float32)
    B, N = Y.shape
    ids = np.empty(B, np.int32)
    lib().orc_argmax(_p(Y), N, N, B, _p(ids))
    return ids


# ---- routing ---------------------------------------------------------------

def router_logits(R, X):
    R = _c(R, np.float32)
    X = _c(np.atleast_2d(X), np.float32)
    E, H = R.shape
    B, ldx = X.shape
    out = np.empty((B, E), np.float64)
    lib().orc_router_logits(_p(R), E, H, _p(X), ldx, B, _p(out))
    return out


def topk(L, k):
    """L: float32 [B, E]; returns int32 [B, k] (descending, lowest index on ties)."""
    L = _c(np.atleast_2d(L), np.float32)
    B, E = L.shape
    ids = np.empty((B, k), np.int32)
    lib().orc_topk(_p(L), E, E, B, k, _p(ids))
    return ids


def gate_weights(logits, ids):
    logits = _c(np.atleast_2d(logits), np.float64)
    ids = _c(np.atleast_2d(ids), np.int32)
    B, k = ids.shape
    w = np.empty((B, k), np.float64)
    lib().orc_gate_weights(_p(logits), logits.shape[1], _p(ids), B, k, _p(w))
    return w


def gather(ids):
    ids = _c(np.atleast_2d(ids), np.int32)
    B, k = ids.shape
    unique = np.empty(B * k, np.int32)
    offsets = np.empty(B * k + 1, np.int32)
    pairs = np.empty(B * k, np.int32)
    U = lib().orc_gather(_p(ids), B, k, _p(unique), _p(offsets), _p(pairs))
    return unique[:U].copy(), offsets[:U + 1].copy(), pairs


# ---- MoE -------------------------------------------------------------------

class MoE:
    """Holds numpy arrays of one MoE layer in the planar Q4_0 layout.

    gate/up: qs uint8 [E, I, H/32, 16], d uint16 [E, I, H/32]
    down:    qs uint8 [E, H, I/32, 16], d uint16 [E, H, I/32]
    shared_*: the same without the leading E (or None).
    """

    def __init__(self, router, gate_qs, gate_d, up_qs, up_d, down_qs, down_d,
                 k, shared=None, shared_gate_row=None):
        self.router = _c(router, np.float32)
        self.E, self.H = self.router.shape
        self.gate_qs, self.gate_d = _c(gate_qs, np.uint8), _c(gate_d, np.uint16)
        self.up_qs, self.up_d = _c(up_qs, np.uint8), _c(up_d, np.uint16)
        self.down_qs, self.down_d = _c(down_qs, np.uint8), _c(down_d, np.uint16)
        self.I = self.gate_qs.shape[1]
        self.k = k
        self.shared = None
        if shared is not None:
            self.shared = tuple(_c(a, np.uint8 if i % 2 == 0 else np.uint16)
                                for i, a in enumerate(shared))
        self.shared_gate_row = (None if shared_gate_row is None
                                else _c(shared_gate_row, np.float32))
        s = _Moe()
        s.E, s.H, s.I, s.k = self.E, self.H, self.I, k
        s.router = _p(self.router).value
        s.shared_gate_row = _p(self.shared_gate_row).value if self.shared_gate_row is not None else None
        s.gate_qs, s.gate_d = _p(self.gate_qs).value, _p(self.gate_d).value
        s.up_qs, s.up_d = _p(self.up_qs).value, _p(self.up_d).value
        s.down_qs, s.down_d = _p(self.down_qs).value, _p(self.down_d).value
        if self.shared is not None:
            gq, gd, uq, ud, dq, dd = self.shared
            s.sh_gate_qs, s.sh_gate_d = _p(gq).value, _p(gd).value
            s.sh_up_qs, s.sh_up_d = _p(uq).value, _p(ud).value
            s.sh_down_qs, s.sh_down_d = _p(dq).value, _p(dd).value
        self._s = s

    @property
    def npairs_per_row(self):
        return self.k + (1 if self.shared is not None else 0)

    def route(self, X):
        X = _c(np.atleast_2d(X), np.float32)
        B = X.shape[0]
        logits = np.empty((B, self.E), np.float64)
        ids = np.empty((B, self.k), np.int32)
        w = np.empty((B, self.k), np.float64)
        s = np.empty(B, np.float64)
        lib().orc_moe_route(C.byref(self._s), _p(X), X.shape[1], B, _p(logits),
                            _p(ids), _p(w), _p(s))
        return logits, ids, w, s

    def gate_up(self, X, ids):
        X = _c(np.atleast_2d(X), np.float32)
        ids = _c(np.atleast_2d(ids), np.int32)
        B = X.shape[0]
        npairs = B * self.k + (B if self.shared is not None else 0)
        h = np.empty((npairs, self.I), np.float32)
        lib().orc_moe_gate_up(C.byref(self._s), _p(X), X.shape[1], B, _p(ids), _p(h))
        return h

    def down(self, hq, hds, ids, w, s):
        hq = _c(hq, np.int8)
        hds = _c(hds, np.uint16)
        ids = _c(np.atleast_2d(ids), np.int32)
        w = _c(np.atleast_2d(w), np.float64)
        s = _c(np.atleast_1d(s), np.float64)
        B = ids.shape[0]
        Y = np.empty((B, self.H), np.float64)
        lib().orc_moe_down(C.byref(self._s), _p(hq), _p(hds), B, _p(ids), _p(w),
                           _p(s), _p(Y))
        return Y

    def layer(self, X):
        """Returns dict(ids, w, s, h, y)."""
        X = _c(np.atleast_2d(X), np.float32)
        B = X.shape[0]
        npairs = B * self.k + (B if self.shared is not None else 0)
        ids = np.empty((B, self.k), np.int32)
        w = np.empty((B, self.k), np.float64)
        s = np.empty(B, np.float64)
        h = np.empty((npairs, self.I), np.float32)
        Y = np.empty((B, self.H), np.float64)
        lib().orc_moe_layer(C.byref(self._s), _p(X), X.shape[1], B, _p(ids), _p(w),
                            _p(s), _p(h), _p(Y))
        return dict(ids=ids, w=w, s=s, h=h, y=Y)
