"""GPU parity of the MoE path (moe_route_topk, moe_mul_mat_id,
moe_layer_decode) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from tests._util import (build_moe, check_ids_admissible, check_route, moe_ref_with_ids, np16,
                         npc, rel_l2_rows)

pytestmark = pytest.mark.gpu

MOE_TOL = 2e-3


def _route_and_check(mm, orc, layer, ref, X):
    ids, w, sw, logits = mm.moe_route_topk(layer.router, X, layer.k,
                                           shared_gate_row=layer.shared_gate_row)
    torch.cuda.synchronize()
    near = check_route(orc, ref.router, npc(X), npc(logits), npc(ids), layer.k, layer.E)
    # weights: softmax renormalised over the selected, from the GPU's ids
    lg_ref = orc.router_logits(ref.router, npc(X))
    w_ref = orc.gate_weights(lg_ref, npc(ids))
    np.testing.assert_allclose(npc(w), w_ref, rtol=2e-5, atol=1e-6)
    if layer.shared_gate_row is not None:
        z = npc(X).astype(np.float64) @ npc(layer.shared_gate_row).astype(np.float64)
        np.testing.assert_allclose(npc(sw), 1 / (1 + np.exp(-z)), rtol=2e-5, atol=1e-6)
    else:
        assert (npc(sw) == 1.0).all()
    return ids, w, sw, near


@pytest.mark.parametrize("E,H,I,k,B,shared,sgate", [
    (16, 256, 64, 4, 1, True, False),
    (16, 256, 64, 4, 8, True, False),
    (64, 512, 96, 6, 3, False, False),
    (40, 256, 32, 16, 8, True, True),
    (256, 2048, 512, 8, 1, True, False),     # the 256-expert decode layer
    (512, 2048, 512, 10, 8, True, False),    # the 512-expert verify batch
    # verify / prefill batches (B > 8): row lists by the counting pass
    (64, 512, 64, 4, 16, True, False),
    (40, 256, 96, 5, 33, False, False),
    (16, 256, 64, 4, 64, True, True),        # every expert chosen by many rows
    (512, 2048, 512, 10, 32, True, False),
])
def test_moe_staged_parity(mm, orc, dev, E, H, I, k, B, shared, sgate):
    layer, ref = build_moe(mm, orc, E, H, I, k, 0, "moe", E, H, I, shared=shared,
                           shared_gate=sgate, device=dev)
    X = synth.activations(B, H, 0, "moe", E, B, device=dev)
    ids, w, sw, _ = _route_and_check(mm, orc, layer, ref, X)

    P = layer.npairs(B)
    nan = lambda *shape: torch.full(shape, np.nan, device=dev)
    dbg = dict(h=nan(P, I), gate_out=nan(P, I), up_out=nan(P, I), down_out=nan(P, H),
               x_q8=torch.full((mm.q8_1_bytes(H, B),), 0xEE, dtype=torch.uint8, device=dev),
               h_q8=torch.full((mm.q8_1_bytes(I, P),), 0xEE, dtype=torch.uint8, device=dev),
               unique=torch.full((B * k,), -1, dtype=torch.int32, device=dev),
               offsets=torch.full((B * k + 1,), -1, dtype=torch.int32, device=dev),
               pairs=torch.full((B * k,), -1, dtype=torch.int32, device=dev),
               n_unique=torch.zeros(1, dtype=torch.int32, device=dev))
    ws = torch.zeros(mm.moe_workspace_bytes(layer, B), dtype=torch.uint8, device=dev)
    y = mm.moe_mul_mat_id(layer, X, ids, w, sw, workspace=ws, debug=dbg)
    torch.cuda.synchronize()
    ids_np = npc(ids)

    # gather lists: bit-exact against the oracle's brute force
    u_ref, o_ref, p_ref = orc.gather(ids_np)
    U = int(npc(dbg["n_unique"])[0])
    assert U == len(u_ref)
    assert np.array_equal(npc(dbg["unique"])[:U], u_ref)
    assert np.array_equal(npc(dbg["offsets"])[:U + 1], o_ref)
    assert np.array_equal(npc(dbg["pairs"]), p_ref)

    # Q8_1(x) as the gate/up workgroups stage it: bit-exact
    xq_ref, xds_ref = orc.quantize_q8_1(npc(X))
    xc, xds = mm.split_q8_1(dbg["x_q8"], B, H)
    assert np.array_equal(npc(xc), xq_ref) and np.array_equal(np16(xds), xds_ref)

    # gate and up of every pair, each against the oracle's W4A8 product on
    # the same Q8_1(x): only the fp32 accumulation order differs
    def mats(p):
        if p < B * k:
            e = int(ids_np.ravel()[p])
            return p // k, (ref.gate_qs[e], ref.gate_d[e]), (ref.up_qs[e], ref.up_d[e]), \
                (ref.down_qs[e], ref.down_d[e])
        gq, gd, uq, ud, dq, dd = ref.shared
        return p - B * k, (gq, gd), (uq, ud), (dq, dd)
    g_gpu, u_gpu = npc(dbg["gate_out"]), npc(dbg["up_out"])
    g_ref = np.empty((P, I))
    u_ref = np.empty((P, I))
    for p in range(P):
        b, (gq, gd), (uq, ud), _ = mats(p)
        g_ref[p] = orc.gemv_q4_0(gq, gd, xq_ref[b:b + 1], xds_ref[b:b + 1])[0]
        u_ref[p] = orc.gemv_q4_0(uq, ud, xq_ref[b:b + 1], xds_ref[b:b + 1])[0]
    assert rel_l2_rows(g_gpu, g_ref) <= 1e-5
    assert rel_l2_rows(u_gpu, u_ref) <= 1e-5

    # h = silu(gate) * up: within tolerance of the oracle (float64 sums)
    h_ref = ref.gate_up(npc(X), ids_np)
    h_gpu = npc(dbg["h"])
    assert rel_l2_rows(h_gpu, h_ref) <= MOE_TOL
    # Q8_1 epilogue, read through the ABI: bit-exact against the oracle
    # quantizer on the GPU's h
    hq_ref, hds_ref = orc.quantize_q8_1(h_gpu)
    hc, hds = mm.split_q8_1(dbg["h_q8"], P, I)
    hq_gpu, hds_gpu = npc(hc), np16(hds)
    assert np.array_equal(hq_gpu, hq_ref)
    assert np.array_equal(hds_gpu, hds_ref)

    # each pair's down product fed the GPU's own Q8_1(h)
    d_gpu = npc(dbg["down_out"])
    for p in range(P):
        _, _, _, (dq, dd) = mats(p)
        d_ref = orc.gemv_q4_0(dq, dd, hq_gpu[p:p + 1], hds_gpu[p:p + 1])[0]
        assert rel_l2_rows(d_gpu[p][None], d_ref[None]) <= 1e-5, p

    # down stage fed the GPU's own Q8_1(h): only fp32 accumulation differs
    w64, s64 = npc(w).astype(np.float64), npc(sw).astype(np.float64)
    y_staged = ref.down(hq_gpu, hds_gpu, ids_np, w64, s64)
    assert rel_l2_rows(npc(y), y_staged) <= 1e-4
    # end to end with the same routing
    hq_o, hds_o = orc.quantize_q8_1(h_ref)
    y_ref = ref.down(hq_o, hds_o, ids_np, w64, s64)
    assert rel_l2_rows(npc(y), y_ref) <= MOE_TOL


@pytest.mark.parametrize("topk_kernel", ["0", "1"])
@pytest.mark.parametrize("E,H,I,k,B", [(256, 2048, 512, 8, 1), (512, 2048, 512, 10, 4),
                                       (32, 512, 64, 4, 8), (20, 96, 64, 3, 2),
                                       (512, 2048, 512, 10, 8), (512, 2048, 512, 10, 16),
                                       (64, 512, 64, 6, 64), (96, 1024, 128, 6, 40)])
def test_moe_layer_decode(mm, orc, dev, path, topk_kernel, E, H, I, k, B):
    # "1": top-k and row lists in a kernel of their own; "0": in every gate/up workgroup
    path(MOE_TOPK=1 if topk_kernel == "1" else -1)
    layer, ref = build_moe(mm, orc, E, H, I, k, 0, "dec", E, H, I, device=dev)
    X = synth.activations(B, H, 0, "dec", E, B, device=dev)
    ids = torch.empty((B, k), dtype=torch.int32, device=dev)
    w = torch.empty((B, k), dtype=torch.float32, device=dev)
    # the workspace needs no initialisation: start from garbage, reuse it
    ws = torch.full((mm.moe_workspace_bytes(layer, B),), 0xA5, dtype=torch.uint8, device=dev)
    y = mm.moe_layer_decode(layer, X, ids=ids, weights=w, workspace=ws)
    y2 = mm.moe_layer_decode(layer, X, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    # every row: ids admissible under fp32 rounding of the logits (rows that
    # differ from the float64 top-k only at near ties), and the output equal
    # to the oracle's for the ids the GPU chose
    ids_np = npc(ids)
    lg64, differ = check_ids_admissible(orc, ref.router, npc(X), ids_np, k)
    assert len(differ) <= max(1, B // 8), differ     # near ties are rare
    y_ref = moe_ref_with_ids(orc, ref, npc(X), ids_np, lg64)
    assert rel_l2_rows(npc(y), y_ref) <= MOE_TOL
    np.testing.assert_allclose(npc(w), orc.gate_weights(lg64, ids_np), rtol=2e-5, atol=1e-6)


@pytest.mark.parametrize("E,H,I,k,B,shared", [
    (1, 32, 32, 1, 1, True),       # one expert, the smallest H and I
    (1, 32, 32, 1, 8, False),
    (4, 64, 32, 4, 3, True),       # k = E: every expert selected
    (16, 256, 64, 16, 8, True),    # k = E = the largest top-k
    (16, 32, 32, 16, 64, True),    # ... at the largest batch
    (8, 32, 64, 1, 64, False),     # k = 1 at the largest batch
])
def test_moe_layer_decode_degenerate(mm, orc, dev, E, H, I, k, B, shared):
    layer, ref = build_moe(mm, orc, E, H, I, k, 0, "degen", E, H, I, shared=shared, device=dev)
    X = synth.activations(B, H, 0, "degen", E, B, device=dev)
    ids = torch.empty((B, k), dtype=torch.int32, device=dev)
    w = torch.empty((B, k), dtype=torch.float32, device=dev)
    y = mm.moe_layer_decode(layer, X, ids=ids, weights=w)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    ids_np = npc(ids)
    lg64, differ = check_ids_admissible(orc, ref.router, npc(X), ids_np, k)
    y_ref = moe_ref_with_ids(orc, ref, npc(X), ids_np, lg64)
    assert rel_l2_rows(npc(y), y_ref) <= MOE_TOL
    np.testing.assert_allclose(npc(w), orc.gate_weights(lg64, ids_np), rtol=2e-5, atol=1e-6)
    if k == E:   # every row selects every expert: weights are the full softmax
        assert np.allclose(npc(w).sum(axis=1), 1.0, atol=1e-5)


@pytest.mark.parametrize("topk_kernel", ["0", "1"])
@pytest.mark.parametrize("B", [1, 2, 5, 12])
def test_moe_layer_decode_tied_router_rows(mm, orc, dev, path, topk_kernel, B):
    # identical router rows give bit-identical logits: the selected experts and
    # their slot order must follow the lower index among equal logits, in the
    # per-workgroup rank selection (one row) as in the full top-k
    path(MOE_TOPK=1 if topk_kernel == "1" else -1)
    E, H, I, k = 64, 512, 64, 8
    t = synth.moe_layer_tensors(E, H, I, 0, "ties", E, device=dev)
    X = synth.activations(B, H, 0, "ties", B, device=dev)
    R = t["router"]
    for b in range(B):  # a strong expert per row, copied to higher and lower indices
        src = 20 + b
        R[src] = 0.3 * X[b] / X[b].norm()
        for dst in (40 + 2 * b, 41 + 2 * b, b):
            R[dst] = R[src]
    sh = t["shared"]
    layer = mm.MoeLayer(R, t["gate_qs"], t["gate_d"], t["up_qs"], t["up_d"], t["down_qs"],
                        t["down_d"], k, shared=sh)
    ref = orc.MoE(npc(R), npc(t["gate_qs"]), np16(t["gate_d"]), npc(t["up_qs"]),
                  np16(t["up_d"]), npc(t["down_qs"]), np16(t["down_d"]), k,
                  shared=tuple(npc(sh[n]) if n.endswith("qs") else np16(sh[n])
                               for n in ("gate_qs", "gate_d", "up_qs", "up_d", "down_qs",
                                         "down_d")))
    ids = torch.empty((B, k), dtype=torch.int32, device=dev)
    y = mm.moe_layer_decode(layer, X, ids=ids)
    torch.cuda.synchronize()
    out = ref.layer(npc(X))
    assert np.array_equal(npc(ids), out["ids"])
    for b in range(B):
        tied = [b, 20 + b, 40 + 2 * b, 41 + 2 * b]
        assert npc(ids)[b, :4].tolist() == tied
    assert rel_l2_rows(npc(y), out["y"]) <= MOE_TOL


def test_topk_exact_ties_from_logits(mm, orc, dev):
    E, k = 300, 10
    g = torch.Generator().manual_seed(3)
    L = torch.randint(-3, 4, (6, E), generator=g).float()      # many exact ties
    L[1] = 0.0
    L[2, 5] = -0.0
    L[2, 9] = 0.0
    ids, w, sw, _ = mm.moe_route_topk(None, L.to(dev), k, n_experts=E)
    torch.cuda.synchronize()
    assert np.array_equal(npc(ids), orc.topk(L.numpy(), k))
    assert np.array_equal(npc(ids)[1], np.arange(k))
    np.testing.assert_allclose(npc(w)[1], np.full(k, 1.0 / k), rtol=1e-6)
    w_ref = orc.gate_weights(L.numpy().astype(np.float64), npc(ids))
    np.testing.assert_allclose(npc(w), w_ref, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("I,B", [(128, 8), (512, 3), (512, 4), (512, 8), (128, 24),
                                 (512, 40)])
def test_moe_batch_invariance(mm, orc, dev, I, B):
    # every row's result has one order whatever the other rows chose: B = 1
    # takes the one-kernel down projection, B >= 3 the by-expert one, B > 8
    # the row-list pass and row groups of eight
    E, H, k = 64, 1024, 6
    layer, _ = build_moe(mm, orc, E, H, I, k, 0, "binv", I, device=dev)
    X = synth.activations(B, H, 0, "binv", device=dev)
    ids, w, sw, _ = mm.moe_route_topk(layer.router, X, k)
    y8 = mm.moe_mul_mat_id(layer, X, ids, w, sw)
    assert torch.equal(y8, mm.moe_mul_mat_id(layer, X, ids, w, sw))
    for b in range(B):
        yb = mm.moe_mul_mat_id(layer, X[b:b + 1].clone(), ids[b:b + 1].clone(),
                               w[b:b + 1].clone(), sw[b:b + 1].clone())
        assert torch.equal(yb, y8[b:b + 1])


def test_moe_single_expert_and_no_shared(mm, orc, dev):
    # k = 1 without a shared expert reduces to one down projection of Q8_1(h)
    E, H, I = 8, 256, 64
    layer, ref = build_moe(mm, orc, E, H, I, 1, 0, "single", shared=False, device=dev)
    X = synth.activations(2, H, 0, "single", device=dev)
    ids = torch.tensor([[3], [6]], dtype=torch.int32, device=dev)
    w = torch.ones((2, 1), device=dev)
    y = mm.moe_mul_mat_id(layer, X, ids, w)
    h = ref.gate_up(npc(X), npc(ids))
    hq, hds = orc.quantize_q8_1(h)
    for b, e in enumerate((3, 6)):
        want = orc.gemv_q4_0(ref.down_qs[e], ref.down_d[e], hq[b:b + 1], hds[b:b + 1])
        assert rel_l2_rows(npc(y)[b:b + 1], want) <= MOE_TOL


@pytest.mark.parametrize("E,H,I,k,shared", [
    (64, 1024, 512, 6, True),     # I = 512: one block per lane
    (32, 512, 1024, 4, True),     # I = 1024: two blocks per lane
    (40, 256, 96, 5, False),      # I = 96: the runtime block loop, no shared expert
    (16, 224, 64, 3, True),       # H not a multiple of 64: a ragged last row tile
])
def test_moe_down_paths_bit_identical(mm, orc, dev, path, E, H, I, k, shared):
    # the by-expert down projection (+ combine) and the one-kernel one form
    # each pair's product and each row's sum in the same order: same bits
    layer, ref = build_moe(mm, orc, E, H, I, k, 0, "dpath", E, H, I, shared=shared, device=dev)
    for B in (1, 2, 3, 8):
        X = synth.activations(B, H, 0, "dpath", E, B, device=dev)
        ids, w, sw, _ = mm.moe_route_topk(layer.router, X, k,
                                          shared_gate_row=layer.shared_gate_row)
        ys = []
        for mode in (1, 2):
            path(MOE_DOWN=mode)
            ws = torch.full((mm.moe_workspace_bytes(layer, B),), 0x5A, dtype=torch.uint8,
                            device=dev)
            ys.append(mm.moe_mul_mat_id(layer, X, ids, w, sw if shared else None, workspace=ws))
        torch.cuda.synchronize()
        assert torch.equal(ys[0], ys[1]), B
        ids_np = npc(ids)
        hq, hds = orc.quantize_q8_1(ref.gate_up(npc(X), ids_np))
        s64 = npc(sw).astype(np.float64) if shared else np.ones(B)
        want = ref.down(hq, hds, ids_np, npc(w).astype(np.float64), s64)
        assert rel_l2_rows(npc(ys[1]), want) <= MOE_TOL


@pytest.mark.parametrize("E,H,B", [(256, 2048, 8), (512, 2048, 40), (64, 1024, 5), (96, 512, 12),
                                   (512, 2048, 31), (160, 1024, 64), (256, 2048, 4),
                                   (512, 2048, 37)])
def test_router_logits_same_bits_for_every_batch(mm, orc, dev, E, H, B):
    # B >= 4 stages x in LDS (H of 1024 or 2048), B < 4 holds it in registers,
    # other H runs the router 8 rows at a time: one fused multiply-add order
    # per lane and one wave sum in every case, so every row's logits are the
    # same bits as the 1-row call's
    t = synth.moe_layer_tensors(E, H, 64, 0, "rbits", E, H, device=dev)
    R, shg = t["router"], synth.normal((H,), 0.02, 0, "rbits-g", E, H, device=dev)
    X = synth.activations(B, H, 0, "rbits", E, B, device=dev)
    k = 4
    _, _, _, lg = mm.moe_route_topk(R, X, k, shared_gate_row=shg)
    for b in range(B):
        _, _, _, lb = mm.moe_route_topk(R, X[b:b + 1].clone(), k, shared_gate_row=shg)
        assert torch.equal(lb[0], lg[b]), b
    torch.cuda.synchronize()
    ref = orc.router_logits(npc(R), npc(X))
    got = npc(lg)[:, :E].astype(np.float64)
    assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-6


def _off2(t):
    # the same values at an address 2 bytes past a 16-byte boundary
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = buf[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("shared", [True, False])
def test_moe_scale_planes_any_alignment(mm, orc, dev, shared):
    # fp16 scale planes 16-byte aligned are read as 16-byte chunks where that
    # pays; planes only 2-byte aligned take per-block loads: the same values,
    # so the same bits
    E, H, I, k = 64, 2048, 512, 6
    layer, ref = build_moe(mm, orc, E, H, I, k, 0, "salign", shared=shared, device=dev)
    t = layer.t
    sh = None
    if shared:
        sh = dict(layer.shared)
        for n in ("gate_d", "up_d", "down_d"):
            sh[n] = _off2(sh[n])
    odd = mm.MoeLayer(layer.router, t["gate_qs"], _off2(t["gate_d"]), t["up_qs"],
                      _off2(t["up_d"]), t["down_qs"], _off2(t["down_d"]), k, shared=sh)
    assert odd.t["gate_d"].data_ptr() % 16 == 2
    for B in (1, 2, 5, 12):
        X = synth.activations(B, H, 0, "salign", B, device=dev)
        ids, w, sw, _ = mm.moe_route_topk(layer.router, X, k)
        sw = sw if shared else None
        y0 = mm.moe_mul_mat_id(layer, X, ids, w, sw)
        y1 = mm.moe_mul_mat_id(odd, X, ids, w, sw)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), B
        ids_np = npc(ids)
        hq, hds = orc.quantize_q8_1(ref.gate_up(npc(X), ids_np))
        s64 = npc(sw).astype(np.float64) if shared else np.ones(B)
        want = ref.down(hq, hds, ids_np, npc(w).astype(np.float64), s64)
        assert rel_l2_rows(npc(y1), want) <= MOE_TOL


@pytest.mark.parametrize("B", [1, 4, 12])
def test_moe_ids_outside_range_add_nothing(mm, orc, dev, B):
    # a pair whose id lies outside [0, E) takes part in no expert list and
    # adds nothing: the same result as its expert kept with weight 0
    E, H, I, k = 64, 1024, 128, 6
    layer, _ = build_moe(mm, orc, E, H, I, k, 0, "badid", B, device=dev)
    X = synth.activations(B, H, 0, "badid", B, device=dev)
    ids, w, sw, _ = mm.moe_route_topk(layer.router, X, k)
    bad, w0 = ids.clone(), w.clone()
    for b in range(B):
        bad[b, 1] = -1 if b % 2 == 0 else E
        w0[b, 1] = 0.0
    y_bad = mm.moe_mul_mat_id(layer, X, bad, w, sw)
    y_ref = mm.moe_mul_mat_id(layer, X, ids, w0, sw)
    torch.cuda.synchronize()
    assert torch.isfinite(y_bad).all()
    assert torch.equal(y_bad, y_ref)


def test_moe_exact_gate_up_and_silu(mm, orc, dev):
    # unit fp16 scales and x = (127, 16, 1, 0, ...): Q8_1(x) has d = 1 and
    # codes x, so every gate output is an exact integer g (chosen per row,
    # from 0 through the bend of the curve to both tails) and every up
    # output is exactly 1.  The staged gate/up outputs must be those integers
    # bit for bit, and h = silu(g) within a few fp32 ulps of scipy's
    # g * expit(g) (the kernel's exp and division round on their own).
    from scipy.special import expit
    from tests.test_oracle_moe import SILU_G
    E, H, I, k = 3, 512, 512, 1
    gate = np.full((E, I, H // 32, 32), 8, np.uint8)
    up = np.full((E, I, H // 32, 32), 8, np.uint8)
    tg = np.array([SILU_G[n % 32] * (1 if n < 256 else -1) for n in range(I)])
    for n, g in enumerate(tg):
        b = (int(g) + 8) // 16
        gate[:, n, 0, 1], gate[:, n, 0, 2] = 8 + b, 8 + (int(g) - 16 * b)
        up[:, n, 0, 2] = 9
    pack = lambda c: torch.from_numpy((c[..., :16] | (c[..., 16:] << 4)).astype(np.uint8)).to(dev)
    ones = lambda *sh: torch.ones(sh, dtype=torch.float16, device=dev)
    down_qs = torch.full((E, H, I // 32, 16), 0x88, dtype=torch.uint8, device=dev)
    router = torch.ones((E, H), device=dev)
    layer = mm.MoeLayer(router, pack(gate), ones(E, I, H // 32), pack(up), ones(E, I, H // 32),
                        down_qs, ones(E, H, I // 32), k)
    X = torch.zeros((2, H), device=dev)
    X[:, :3] = torch.tensor([127.0, 16.0, 1.0])
    ids = torch.tensor([[1], [2]], dtype=torch.int32, device=dev)
    w = torch.ones((2, 1), device=dev)
    P = 2
    dbg = dict(gate_out=torch.full((P, I), np.nan, device=dev),
               up_out=torch.full((P, I), np.nan, device=dev),
               h=torch.full((P, I), np.nan, device=dev))
    y = mm.moe_mul_mat_id(layer, X, ids, w, debug=dbg)
    torch.cuda.synchronize()
    for p in range(P):
        assert np.array_equal(npc(dbg["gate_out"])[p], tg.astype(np.float32))
        assert (npc(dbg["up_out"])[p] == 1.0).all()
        want = (tg * expit(tg)).astype(np.float32)
        h = npc(dbg["h"])[p].astype(np.float64)
        assert (np.abs(h - want) <= 4 * np.spacing(np.abs(want)) + 1e-30).all()
    assert (npc(y) == 0.0).all()        # all-zero down weights (codes 8)


def _strided(t, extra, fill):
    """t [E, ...] as a view into a padded stack: each expert's bytes followed
    by `extra` elements of `fill` (never read when the strides are right)."""
    E, n = t.shape[0], t[0].numel()
    big = torch.empty((E, n + extra), dtype=t.dtype, device=t.device)
    big.view(torch.uint8).fill_(fill)
    big[:, :n] = t.reshape(E, n)
    v = big[:, :n].view(t.shape)
    assert v.stride(0) == n + extra and v[0].is_contiguous()
    return v


@pytest.mark.gpu
@pytest.mark.parametrize("d_extra", [3, 8])      # 8: scale planes stay 16-byte aligned
@pytest.mark.parametrize("B", [1, 2, 5, 16])
def test_moe_expert_strides(mm, orc, dev, d_extra, B):
    # experts with padding between them (layer-level expert strides) give the
    # bits of the contiguous stack on every launch path
    E, H, I, k = 64, 1024, 512, 6
    t = synth.moe_layer_tensors(E, H, I, 0, "strides", shared=True, device=dev)
    base = mm.MoeLayer(t["router"], t["gate_qs"], t["gate_d"], t["up_qs"], t["up_d"],
                       t["down_qs"], t["down_d"], k, shared=t["shared"])
    v = {name: _strided(t[name], 48 if name.endswith("qs") else d_extra, 0xFF)
         for name in ("gate_qs", "gate_d", "up_qs", "up_d", "down_qs", "down_d")}
    lay = mm.MoeLayer(t["router"], v["gate_qs"], v["gate_d"], v["up_qs"], v["up_d"],
                      v["down_qs"], v["down_d"], k, shared=t["shared"])
    assert lay._s.gate_qs_stride == I * H // 2 + 48 and lay._s.down_d_stride == H * I // 32 + d_extra
    X = synth.activations(B, H, 0, "strides", B, device=dev)
    y0 = mm.moe_layer_decode(base, X)
    y1 = mm.moe_layer_decode(lay, X)
    torch.cuda.synchronize()
    assert torch.isfinite(y1).all()
    assert torch.equal(y0, y1)
