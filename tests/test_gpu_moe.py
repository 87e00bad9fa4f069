"""GPU parity of the MoE path (moe_route_topk, moe_mul_mat_id,
moe_layer_decode) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from tests._util import build_moe, check_route, np16, npc, rel_l2_rows

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
    dbg = dict(h=torch.full((P, I), np.nan, device=dev),
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

    # gate/up stage: h within tolerance of the oracle (float64 sums)
    h_ref = ref.gate_up(npc(X), ids_np)
    h_gpu = npc(dbg["h"])
    assert rel_l2_rows(h_gpu, h_ref) <= MOE_TOL
    # Q8_1 epilogue: bit-exact against the oracle quantizer on the GPU's h
    hq_ref, hds_ref = orc.quantize_q8_1(h_gpu)
    raw = npc(ws)
    hq_gpu = raw[:P * I].view(np.int8).reshape(P, I)
    hds_gpu = raw[P * I:P * I + 4 * P * (I // 32)].view(np.uint16).reshape(P, I // 32, 2)
    assert np.array_equal(hq_gpu, hq_ref)
    assert np.array_equal(hds_gpu, hds_ref)

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
def test_moe_layer_decode(mm, orc, dev, monkeypatch, topk_kernel, E, H, I, k, B):
    # "1": top-k and row lists in a kernel of their own; "0": in every gate/up workgroup
    monkeypatch.setenv("MMV_MOE_TOPK_KERNEL", topk_kernel)
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
    out = ref.layer(npc(X))
    same = [b for b in range(B) if np.array_equal(npc(ids)[b], out["ids"][b])]
    assert len(same) >= B - 1            # near ties in float64 logits are rare
    assert rel_l2_rows(npc(y)[same], out["y"][same]) <= MOE_TOL


@pytest.mark.parametrize("topk_kernel", ["0", "1"])
@pytest.mark.parametrize("B", [1, 2, 5, 12])
def test_moe_layer_decode_tied_router_rows(mm, orc, dev, monkeypatch, topk_kernel, B):
    # identical router rows give bit-identical logits: the selected experts and
    # their slot order must follow the lower index among equal logits, in the
    # per-workgroup rank selection (one row) as in the full top-k
    monkeypatch.setenv("MMV_MOE_TOPK_KERNEL", topk_kernel)
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
def test_moe_down_paths_bit_identical(mm, orc, dev, monkeypatch, E, H, I, k, shared):
    # the by-expert down projection (+ combine) and the one-kernel one form
    # each pair's product and each row's sum in the same order: same bits
    layer, ref = build_moe(mm, orc, E, H, I, k, 0, "dpath", E, H, I, shared=shared, device=dev)
    for B in (1, 2, 3, 8):
        X = synth.activations(B, H, 0, "dpath", E, B, device=dev)
        ids, w, sw, _ = mm.moe_route_topk(layer.router, X, k,
                                          shared_gate_row=layer.shared_gate_row)
        ys = []
        for mode in ("1", "2"):
            monkeypatch.setenv("MMV_MOE_DOWN", mode)
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
