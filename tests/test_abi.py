"""The C-ABI library loads, exports every function include/moe_matvec.h
declares, and rejects bad arguments on the host before any launch.

Every call here fails validation, so nothing touches a device: pointers are
fake addresses chosen only for their alignment and ranges."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in sorted(os.listdir(os.path.join(ROOT, "include")))
           if n.endswith(".h")]

OK, E_NULL, E_SHAPE, E_ALIGN, E_BATCH, E_TOPK, E_WS, E_ALIAS, E_HIP, E_ARG = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def L():
    import moe_matvec_amd
    return moe_matvec_amd.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert {"gemv_bf16", "gemv_q4_0", "quantize_q8_1", "moe_route_topk",
            "moe_mul_mat_id"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in (OK, E_NULL, E_SHAPE, E_ALIGN, E_BATCH, E_TOPK, E_WS, E_ALIAS, E_HIP, E_ARG):
        assert L.mmv_status_str(s) and L.mmv_status_str(s) != b"unknown status"
    assert L.mmv_status_str(5) == b"unknown status"
    assert L.mmv_last_hip_error() == 0
    assert L.mmv_q8_1_bytes(4096, 8) == 8 * 4096 + 4 * 8 * 128
    assert L.mmv_q8_1_bytes(33, 1) == 0


A = 0x10000000      # 256-byte aligned fake device addresses, far apart
Bp = 0x20000000
Cp = 0x30000000
Dp = 0x40000000


def test_gemv_bf16_validation(L):
    g = L.gemv_bf16
    assert g(None, 8, 64, 64, Bp, 64, 1, Cp, 8, None) == E_NULL
    assert g(A, 8, 64, 64, Bp, 64, 0, Cp, 8, None) == E_BATCH
    assert g(A, 8, 64, 64, Bp, 64, 9, Cp, 8, None) == E_BATCH
    assert g(A, 8, 60, 64, Bp, 64, 1, Cp, 8, None) == E_SHAPE     # K % 8
    assert g(A, 0, 64, 64, Bp, 64, 1, Cp, 8, None) == E_SHAPE     # N
    assert g(A, 8, 64, 56, Bp, 64, 1, Cp, 8, None) == E_SHAPE     # ldw < K
    assert g(A, 8, 64, 64, Bp, 64, 2, Cp, 4, None) == E_SHAPE     # ldy < N
    assert g(A + 2, 8, 64, 64, Bp, 64, 1, Cp, 8, None) == E_ALIGN
    assert g(A, 8, 64, 68, Bp, 64, 1, Cp, 8, None) == E_ALIGN     # ldw % 8
    assert g(A, 8, 64, 64, Bp + 4, 64, 1, Cp, 8, None) == E_ALIGN
    assert g(A, 8, 64, 64, Bp, 66, 2, Cp, 8, None) == E_ALIGN     # ldx % 4
    assert g(A, 8, 64, 64, Bp, 64, 1, A + 64, 8, None) == E_ALIAS  # y inside W
    assert g(A, 8, 64, 64, Bp, 64, 2, Bp + 200, 8, None) == E_ALIAS


def test_quantize_validation(L):
    q = L.quantize_q8_1
    assert q(None, 64, 64, 1, Bp, None) == E_NULL
    assert q(A, 48, 64, 1, Bp, None) == E_SHAPE
    assert q(A, 64, 32, 1, Bp, None) == E_SHAPE
    assert q(A, 64, 64, 9, Bp, None) == E_BATCH
    assert q(A, 64, 64, 1, Bp + 8, None) == E_ALIGN
    assert q(A, 64, 64, 1, A + 128, None) == E_ALIAS


def _q4(qs, d, N, K):
    import moe_matvec_amd as m
    return m._Q4(qs, d, N, K)


def test_gemv_q4_0_validation(L):
    g = L.gemv_q4_0
    W = _q4(A, Bp, 64, 256)
    assert g(None, Cp, 256, None, 1, Dp, 64, None) == E_NULL
    assert g(C.byref(W), None, 256, None, 1, Dp, 64, None) == E_NULL  # neither X nor Xq
    # X and Xq both given: Xq is an output and must not overlap X, Y or W
    assert g(C.byref(W), Cp, 256, Cp + 512, 1, Dp, 64, None) == E_ALIAS
    assert g(C.byref(W), Cp, 256, Dp + 128, 1, Dp, 64, None) == E_ALIAS
    assert g(C.byref(W), Cp, 256, A + 256, 1, Dp, 64, None) == E_ALIAS
    assert g(C.byref(W), Cp, 256, None, 0, Dp, 64, None) == E_BATCH
    assert g(C.byref(_q4(A, Bp, 64, 200)), Cp, 256, None, 1, Dp, 64, None) == E_SHAPE
    assert g(C.byref(_q4(A, Bp, 64, 32 * 1600)), Cp, 51200, None, 8, Dp, 64, None) == E_SHAPE
    assert g(C.byref(_q4(A + 8, Bp, 64, 256)), Cp, 256, None, 1, Dp, 64, None) == E_ALIGN
    assert g(C.byref(_q4(A, Bp + 1, 64, 256)), Cp, 256, None, 1, Dp, 64, None) == E_ALIGN
    assert g(C.byref(W), None, 0, Cp + 4, 1, Dp, 64, None) == E_ALIGN
    assert g(C.byref(W), Cp, 256, None, 1, A + 16, 64, None) == E_ALIAS
    assert g(C.byref(W), Cp, 256, None, 1, Bp + 4, 64, None) == E_ALIAS


def test_route_validation(L):
    r = L.moe_route_topk
    args = dict(router=A, E=256, H=2048, X=Bp, ldx=2048, B=1, k=8, shg=None,
                logits=Cp, ids=Dp, weights=Dp + 4096, sw=Dp + 8192)

    def call(**kw):
        a = dict(args, **kw)
        return r(a["router"], a["E"], a["H"], a["X"], a["ldx"], a["B"], a["k"], a["shg"],
                 a["logits"], a["ids"], a["weights"], a["sw"], None)
    assert call(ids=None) == E_NULL
    assert call(logits=None) == E_NULL
    assert call(B=0) == E_BATCH
    assert call(B=65) == E_BATCH                      # MMV_MOE_MAX_BATCH = 64
    assert call(E=0) == E_SHAPE
    assert call(E=1025) == E_SHAPE
    assert call(k=0) == E_TOPK
    assert call(k=17) == E_TOPK
    assert call(E=4, k=5) == E_TOPK
    assert call(router=None, shg=A + 0x100000) == E_ARG
    assert call(H=2046) == E_SHAPE
    assert call(ldx=1024) == E_SHAPE
    assert call(X=Bp + 4) == E_ALIGN
    assert call(ids=Dp + 2) == E_ALIGN
    assert call(ids=Cp + 64) == E_ALIAS                 # ids inside logits
    assert call(weights=Dp + 16) == E_ALIAS             # weights overlap ids
    assert call(logits=A + 64) == E_ALIAS               # logits inside router


def _layer(**over):
    import moe_matvec_amd as m
    s = m._Layer()
    s.n_experts, s.hidden, s.inter, s.top_k = 256, 2048, 512, 8
    base = 0x1000000000
    for i, name in enumerate(["router", "gate_qs", "up_qs", "down_qs", "gate_d", "up_d",
                              "down_d"]):
        setattr(s, name, base + i * 0x100000000)
    for k, v in over.items():
        setattr(s, k, v)
    return s


def test_mul_mat_id_validation(L):
    f = L.moe_mul_mat_id
    X, ids, w, Y, ws = A, Bp, Bp + 0x1000, Cp, Dp
    lay = _layer()
    need = L.moe_workspace_bytes(C.byref(lay), 1)
    assert need > 0

    def call(layer=lay, B=1, ws_bytes=need, **kw):
        a = dict(X=X, ids=ids, w=w, sw=None, Y=Y, ws=ws, ldx=2048, ldy=2048)
        a.update(kw)
        return f(C.byref(layer), a["X"], a["ldx"], B, a["ids"], a["w"], a["sw"], a["Y"],
                 a["ldy"], a["ws"], ws_bytes, None, None)
    assert call(ws_bytes=need - 1) == E_WS
    assert call(ws=None) == E_WS
    assert call(ws=Dp + 16) == E_ALIGN
    assert call(B=65) == E_BATCH
    assert call(B=8) == E_WS                               # workspace sized for B = 1
    assert call(B=64) == E_WS                              # verify / prefill batches
    assert call(ids=None) == E_NULL
    assert call(layer=_layer(top_k=17)) == E_TOPK
    assert call(layer=_layer(inter=500)) == E_SHAPE
    assert call(layer=_layer(gate_qs=None)) == E_NULL
    assert call(layer=_layer(sh_gate_qs=0x5000000000)) == E_ARG   # partial shared expert
    assert call(layer=_layer(down_qs=0x1300000008)) == E_ALIGN
    assert call(ldx=1000) == E_SHAPE
    assert call(Y=ws + 64) == E_ALIAS
    assert call(Y=0x1000000000 + 64) == E_ALIAS            # output inside the router
    assert call(ws=X) == E_ALIAS


def test_layer_expert_strides(L):
    # strides between routed experts: 0 = contiguous, else at least one
    # expert's plane (qs: a multiple of 16 bytes); the alias check covers
    # the strided extent
    f = L.moe_mul_mat_id
    one_qs, one_d = 512 * 2048 // 2, 512 * 2048 // 32   # one expert's planes (I = 512, H = 2048)

    def call(layer, Y=Cp):
        need = L.moe_workspace_bytes(C.byref(layer), 1)
        return f(C.byref(layer), A, 2048, 1, Bp, Bp + 0x1000, None, Y, 2048, Dp,
                 max(need, 1 << 20), None, None)
    for name, bad in (("gate_qs_stride", one_qs - 16), ("up_qs_stride", one_qs + 8),
                      ("down_qs_stride", -16), ("gate_d_stride", one_d - 1),
                      ("down_d_stride", -1), ("up_d_stride", 1 << 41)):
        lay = _layer(**{name: bad})
        assert L.moe_workspace_bytes(C.byref(lay), 1) == 0, name
        assert call(lay) == E_SHAPE, name
    for name, good in (("gate_qs_stride", one_qs + 16), ("down_qs_stride", 1 << 20),
                       ("up_d_stride", one_d + 1), ("down_d_stride", 2 * one_d)):
        assert L.moe_workspace_bytes(C.byref(_layer(**{name: good})), 1) > 0, name
    # an output 160 MB into gate_qs: past 256 contiguous experts (128 MB),
    # inside them at a 1 MB stride (every call here must fail validation, so
    # the contiguous case, which would pass it, is not called)
    Y = 0x1100000000 + 0xA000000
    assert call(_layer(gate_qs_stride=1 << 20), Y=Y) == E_ALIAS
    assert call(_layer(down_d_stride=1 << 24), Y=0x1600000000 + (1 << 32)) == E_ALIAS


def test_layer_decode_validation(L):
    f = L.moe_layer_decode
    lay = _layer()
    need = L.moe_workspace_bytes(C.byref(lay), 2)
    assert f(C.byref(lay), A, 2048, 2, Cp, 2048, None, None, Dp, need - 256, None) == E_WS
    assert f(C.byref(lay), None, 2048, 2, Cp, 2048, None, None, Dp, need, None) == E_NULL
    assert f(C.byref(lay), A, 2048, 2, Cp, 2048, A + 8, None, Dp, need, None) == E_ALIAS
    assert f(C.byref(lay), A, 2048, 2, Cp, 2048, Dp + 64, None, Dp, need, None) == E_ALIAS


def test_gemv_q4_0_f32_validation(L):
    g = L.gemv_q4_0_f32
    W = _q4(A, Bp, 64, 512)
    assert g(None, Cp, 512, 1, Dp, 64, None) == E_NULL
    assert g(C.byref(W), None, 512, 1, Dp, 64, None) == E_NULL
    assert g(C.byref(W), Cp, 512, 0, Dp, 64, None) == E_BATCH
    assert g(C.byref(_q4(A, Bp, 64, 80)), Cp, 96, 1, Dp, 64, None) == E_SHAPE    # K % 32
    assert g(C.byref(_q4(A, Bp, 64, 8192)), Cp, 8192, 5, Dp, 64, None) == E_SHAPE  # B*K
    assert g(C.byref(_q4(A, Bp, 64, 36896)), Cp, 36896, 1, Dp, 64, None) == E_SHAPE
    assert g(C.byref(W), Cp, 500, 1, Dp, 64, None) == E_SHAPE                  # ldx < K
    assert g(C.byref(W), Cp + 4, 512, 1, Dp, 64, None) == E_ALIGN
    assert g(C.byref(W), Cp, 514, 2, Dp, 64, None) == E_ALIGN                  # ldx % 4
    assert g(C.byref(W), Cp, 512, 1, A + 64, 64, None) == E_ALIAS
    assert g(C.byref(W), Cp, 512, 1, Cp + 16, 64, None) == E_ALIAS


def test_argmax_validation(L):
    a = L.argmax_rows
    assert L.mmv_argmax_workspace_bytes(248320, 8) == 8 * 61 * 8
    assert L.mmv_argmax_workspace_bytes(0, 1) == 0
    ws = L.mmv_argmax_workspace_bytes(5000, 2)
    assert a(None, 5000, 5000, 2, Bp, Cp, Dp, ws, None) == E_NULL
    assert a(A, 5000, 5000, 2, None, Cp, Dp, ws, None) == E_NULL
    assert a(A, 5000, 5000, 2, Bp, None, None, ws, None) == E_NULL             # workspace
    assert a(A, 5000, 5000, 9, Bp, Cp, Dp, ws, None) == E_BATCH
    assert a(A, 4000, 5000, 2, Bp, Cp, Dp, ws, None) == E_SHAPE                # ldy < N
    assert a(A, 5000, 0, 2, Bp, Cp, Dp, ws, None) == E_SHAPE
    assert a(A + 2, 5000, 5000, 2, Bp, Cp, Dp, ws, None) == E_ALIGN
    assert a(A, 5000, 5000, 2, Bp, Cp, Dp + 4, ws, None) == E_ALIGN
    assert a(A, 5000, 5000, 2, Bp, Cp, Dp, ws - 8, None) == E_WS
    assert a(A, 5000, 5000, 2, A + 40, Cp, Dp, ws, None) == E_ALIAS            # ids inside Y
    assert a(A, 5000, 5000, 2, Bp, Bp + 4, Dp, ws, None) == E_ALIAS            # vals on ids
    assert a(A, 5000, 5000, 2, Bp, Cp, A + 1024, ws, None) == E_ALIAS          # ws inside Y


def test_large_pair_count_times_inter_is_accepted(L):
    # Q8_1(h) of P = B*k (+B) pairs times I no longer bounds the MoE calls: the
    # down projection stages it on chip only where it fits and otherwise runs
    # by expert.  Validation passes the shape checks and stops at the
    # (deliberately short) workspace, so nothing is launched.
    big = _layer(top_k=16, inter=1024)
    for B in (1, 2, 3, 6, 8):
        need = L.moe_workspace_bytes(C.byref(big), B)
        assert need > 0
        r = L.moe_mul_mat_id(C.byref(big), A, 2048, B, Bp, Bp + 0x1000, None, Cp, 2048, Dp,
                             need - 1, None, None)
        assert r == E_WS, B
        r = L.moe_layer_decode(C.byref(big), A, 2048, B, Cp, 2048, None, None, Dp, need - 1,
                               None)
        assert r == E_WS, B


def test_path_switches(L):
    # the test-only variant switches: set returns the previous value, unknown
    # switches are refused, and everything returns to automatic (0)
    assert L.mmv_get_path(7) == 0
    assert L.mmv_set_path(7, 1) == 0
    assert L.mmv_get_path(7) == 1
    assert L.mmv_set_path(7, 0) == 1
    assert L.mmv_set_path(99, 1) == E_ARG and L.mmv_set_path(-1, 1) == E_ARG
    assert L.mmv_get_path(99) == 0
    import moe_matvec_amd as m
    n = len(m.PATH)
    assert sorted(m.PATH.values()) == list(range(n))
    assert L.mmv_set_path(n, 1) == E_ARG                   # one past the last switch
    for i in range(n):
        assert L.mmv_get_path(i) == 0


def test_noalloc_refuses_oversized_layers(L):
    # the library's own workspace: its size is exported, and a layer whose
    # workspace exceeds it is refused before any device call
    assert L.mmv_noalloc_ws_bytes() == 8 << 20
    big = _layer(n_experts=1024, hidden=4096, inter=1024, top_k=16)
    assert L.moe_workspace_bytes(C.byref(big), 64) > L.mmv_noalloc_ws_bytes()
    assert L.moe_layer_decode_noalloc(C.byref(big), A, 4096, 64, Cp, 4096, None, None,
                                      None) == E_WS
    assert L.moe_layer_decode_noalloc(None, A, 2048, 1, Cp, 2048, None, None, None) == E_NULL
    assert L.moe_layer_decode_noalloc(C.byref(_layer()), A, 2048, 0, Cp, 2048, None, None,
                                      None) == E_BATCH
    assert L.moe_layer_decode_noalloc(C.byref(_layer(top_k=17)), A, 2048, 1, Cp, 2048, None,
                                      None, None) == E_TOPK


def test_stream_read_validation(L):
    s = L.mmv_stream_read
    n = L.mmv_probe_slots()
    assert n > 0
    assert s(None, 1 << 20, Bp, None) == E_NULL
    assert s(A, 1 << 20, None, None) == E_NULL
    assert s(A, 8, Bp, None) == E_SHAPE
    assert s(A, (1 << 20) + 8, Bp, None) == E_SHAPE
    assert s(A, (1 << 38) + 16, Bp, None) == E_SHAPE        # one dispatch's work-item count
    assert s(A + 8, 1 << 20, Bp, None) == E_ALIGN
    assert s(A, 1 << 20, Bp + 2, None) == E_ALIGN
    assert s(A, 1 << 20, A + 64, None) == E_ALIAS


def test_timeline_absent_from_the_normal_build(L):
    # only the separate timeline build notes timestamps; the product library
    # answers 0 without touching a device
    assert L.mmv_timeline(None, 0, None) == 0
    assert L.mmv_timeline(None, 1, None) == 0
