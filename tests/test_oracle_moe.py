"""Pins of the oracle's router, top-k, gate weights, gather lists and whole MoE
layer: numpy matmuls, a stable sort on (-value, index), Python's sorted(),
closed forms, scipy's logistic function for the SiLU between gate and up, and
a dense numpy restatement of the layer on small cases."""
import numpy as np
import pytest
from scipy.special import expit

from tests.test_oracle_gemv import _dense_q4, _q8_dense


def test_router_logits_match_numpy(orc):
    rng = np.random.default_rng(10)
    R = (rng.standard_normal((40, 96)) * 0.02).astype(np.float32)
    X = rng.standard_normal((3, 96)).astype(np.float32)
    np.testing.assert_allclose(orc.router_logits(R, X), X.astype(np.float64) @ R.T.astype(np.float64),
                               rtol=1e-13, atol=1e-15)


def _topk_ref(L, k):
    # stable lexicographic order on (-value, index)
    out = []
    for row in L:
        order = np.lexsort((np.arange(row.size), -row.astype(np.float64)))
        out.append(order[:k])
    return np.array(out, np.int32)


@pytest.mark.parametrize("E,k", [(8, 1), (8, 8), (256, 8), (512, 10), (1000, 16)])
def test_topk_matches_sort(orc, E, k):
    rng = np.random.default_rng(E + k)
    L = rng.standard_normal((5, E)).astype(np.float32)
    # plant exact ties, including one straddling the k / k+1 boundary
    L[1, :] = np.round(L[1, :] * 2) / 2
    L[2, :] = 0.0
    L[3, 7 % E] = L[3, 3 % E] = L[3].max() + 1.0
    assert np.array_equal(orc.topk(L, k), _topk_ref(L, k))


def test_topk_special_cases(orc):
    L = np.zeros((1, 16), np.float32)
    assert np.array_equal(orc.topk(L, 4)[0], [0, 1, 2, 3])          # all equal: lowest ids
    L = np.array([[1.0, 3.0, 3.0, 2.0, -0.0, 0.0]], np.float32)
    assert np.array_equal(orc.topk(L, 6)[0], [1, 2, 3, 0, 4, 5])    # -0 == +0: index order
    assert orc.topk(L, 1)[0, 0] == 1                                  # argmax, lowest index


def test_gate_weights_closed_forms(orc):
    lg = np.zeros((1, 32))
    w = orc.gate_weights(lg, orc.topk(lg.astype(np.float32), 8))
    assert np.array_equal(w, np.full((1, 8), 0.125))
    # k = E: the full softmax
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((2, 10))
    ids = orc.topk(lg.astype(np.float32), 10)
    w = orc.gate_weights(lg, ids)
    sm = np.exp(lg - lg.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(sm, ids, 1), rtol=1e-14)
    # renormalised over the selected: equals softmax-then-renormalise
    ids = orc.topk(lg.astype(np.float32), 3)
    w = orc.gate_weights(lg, ids)
    p = np.take_along_axis(sm, ids, 1)
    np.testing.assert_allclose(w, p / p.sum(1, keepdims=True), rtol=1e-14)
    assert np.allclose(w.sum(1), 1.0)


def test_gather_matches_sorted(orc):
    rng = np.random.default_rng(12)
    for B, k, E in [(1, 8, 256), (8, 10, 512), (8, 16, 20), (4, 3, 3)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(B)]).astype(np.int32)
        unique, offsets, pairs = orc.gather(ids)
        entries = sorted((int(ids[b, j]), b, j) for b in range(B) for j in range(k))
        assert list(unique) == sorted(set(ids.ravel().tolist()))
        assert [b * k + j for (_, b, j) in entries] == list(pairs)
        for u, e in enumerate(unique):
            assert all(ids.ravel()[p] == e for p in pairs[offsets[u]:offsets[u + 1]])
        assert offsets[-1] == B * k
        if B == 1:
            assert list(unique) == sorted(ids[0].tolist())


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def _rand_layer(orc, rng, E, H, I, k, shared=True, shared_gate=False, scale=0.02):
    def q4(n_mat, N, K):
        codes = rng.integers(0, 16, size=(n_mat, N, K // 32, 32)).astype(np.uint8)
        qs = (codes[..., :16] | (codes[..., 16:] << 4)).astype(np.uint8)
        d = (rng.random((n_mat, N, K // 32)) * scale / 8 + scale / 64).astype(np.float16).view(np.uint16)
        return qs, d
    router = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    gq, gd = q4(E, I, H)
    uq, ud = q4(E, I, H)
    dq, dd = q4(E, H, I)
    sh = None
    if shared:
        a, b = q4(1, I, H)
        c, d = q4(1, I, H)
        e, f = q4(1, H, I)
        sh = (a[0], b[0], c[0], d[0], e[0], f[0])
    sgr = (rng.standard_normal(H) * 0.05).astype(np.float32) if shared_gate else None
    return orc.MoE(router, gq, gd, uq, ud, dq, dd, k, shared=sh, shared_gate_row=sgr)


def _dense_layer(orc, L, X):
    """Dense numpy restatement: decoded matrices, numpy matmuls."""
    B = X.shape[0]
    logits = X.astype(np.float64) @ L.router.astype(np.float64).T
    ids = _topk_ref(logits.astype(np.float32), L.k)
    sel = np.take_along_axis(logits, ids, 1)
    w = np.exp(sel - sel.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    if L.shared_gate_row is not None:
        s = 1 / (1 + np.exp(-(X.astype(np.float64) @ L.shared_gate_row.astype(np.float64))))
    else:
        s = np.ones(B)
    xq, xds = orc.quantize_q8_1(X)
    xhat = _q8_dense(xq, xds)
    silu = lambda z: z * expit(z)   # scipy's logistic function, not the oracle's formula
    Y = np.zeros((B, L.H))
    for b in range(B):
        experts = [(int(ids[b, j]), w[b, j], False) for j in range(L.k)]
        if L.shared is not None:
            experts.append((None, s[b], True))
        for e, wt, is_sh in experts:
            if is_sh:
                gq, gd, uq, ud, dq, dd = L.shared
            else:
                gq, gd, uq, ud, dq, dd = (L.gate_qs[e], L.gate_d[e], L.up_qs[e], L.up_d[e],
                                          L.down_qs[e], L.down_d[e])
            g = _dense_q4(gq, gd) @ xhat[b]
            u = _dense_q4(uq, ud) @ xhat[b]
            h = (silu(g) * u).astype(np.float32)
            hq, hds = orc.quantize_q8_1(h[None])
            Y[b] += wt * (_dense_q4(dq, dd) @ _q8_dense(hq, hds)[0])
    return ids, w, s, Y


@pytest.mark.parametrize("shared,shared_gate", [(True, False), (False, False), (True, True)])
def test_layer_matches_dense_restatement(orc, shared, shared_gate):
    rng = np.random.default_rng(13)
    L = _rand_layer(orc, rng, E=12, H=64, I=64, k=3, shared=shared, shared_gate=shared_gate)
    X = rng.standard_normal((4, 64)).astype(np.float32)
    out = orc.MoE.layer(L, X)
    ids, w, s, Y = _dense_layer(orc, L, X)
    assert np.array_equal(out["ids"], ids)
    np.testing.assert_allclose(out["w"], w, rtol=1e-13)
    np.testing.assert_allclose(out["s"], s, rtol=1e-13)
    np.testing.assert_allclose(out["y"], Y, rtol=1e-9, atol=1e-12)


def test_layer_single_expert_reduces_to_down(orc):
    rng = np.random.default_rng(14)
    L = _rand_layer(orc, rng, E=5, H=64, I=32, k=1, shared=False)
    X = rng.standard_normal((2, 64)).astype(np.float32)
    out = L.layer(X)
    assert np.array_equal(out["w"], np.ones((2, 1)))
    for b in range(2):
        e = out["ids"][b, 0]
        hq, hds = orc.quantize_q8_1(out["h"][b][None])
        y = orc.gemv_q4_0(L.down_qs[e], L.down_d[e], hq, hds)[0]
        assert np.array_equal(out["y"][b], y)


def test_layer_identical_experts_weights_sum_to_one(orc):
    rng = np.random.default_rng(15)
    L1 = _rand_layer(orc, rng, E=1, H=64, I=32, k=1, shared=False)
    E = 6
    rep = lambda a: np.repeat(a, E, axis=0)
    router = (rng.standard_normal((E, 64))).astype(np.float32)
    L = orc.MoE(router, rep(L1.gate_qs), rep(L1.gate_d), rep(L1.up_qs), rep(L1.up_d),
                rep(L1.down_qs), rep(L1.down_d), 4)
    X = rng.standard_normal((3, 64)).astype(np.float32)
    y1 = L1.layer(X)["y"]
    y = L.layer(X)["y"]
    np.testing.assert_allclose(y, y1, rtol=1e-12, atol=1e-14)


def test_layer_zero_gate_gives_zero(orc):
    rng = np.random.default_rng(16)
    L0 = _rand_layer(orc, rng, E=4, H=32, I=32, k=2, shared=True)
    gd = np.zeros_like(L0.gate_d)
    L = orc.MoE(L0.router, L0.gate_qs, gd, L0.up_qs, L0.up_d, L0.down_qs, L0.down_d, 2,
                shared=(L0.shared[0], np.zeros_like(L0.shared[1])) + L0.shared[2:])
    out = L.layer(rng.standard_normal((2, 32)).astype(np.float32))
    assert not out["h"].any() and not out["y"].any()


def test_batched_rows_equal_single_rows(orc):
    rng = np.random.default_rng(17)
    L = _rand_layer(orc, rng, E=16, H=64, I=32, k=4, shared=True)
    X = rng.standard_normal((8, 64)).astype(np.float32)
    full = L.layer(X)
    for b in range(8):
        one = L.layer(X[b:b + 1])
        assert np.array_equal(one["ids"][0], full["ids"][b])
        assert np.array_equal(one["y"][0], full["y"][b])


# ---------------------------------------------------------------------------
# SiLU between gate and up, reached through the layer's gate/up stage
# ---------------------------------------------------------------------------

# gate outputs g driven to exact integers (below): 0, the small values where
# the curve bends, and the tails where silu(g) -> g (g -> +inf) and
# silu(g) -> 0 from below (g -> -inf)
SILU_G = [0, 1, -1, 2, -2, 3, -3, 5, -5, 8, -8, 10, -10, 17, -17, 20, -20, 30, -30,
          40, -40, 60, -60, 88, -88, 100, -100, 119, -119, 50, -50, 7]


def _silu_layer(orc, targets):
    """One expert, H = I = 32, unit fp16 scales.  x = (127, 16, 1, 0, ...)
    quantizes to exactly those codes with d = 1 (amax = 127).  Gate row n has
    codes (8, 8 + b_n, 8 + c_n, 8, ...) with 16 b_n + c_n = target n, so
    g_n = 16 b_n + c_n exactly; every up row has codes (8, 8, 9, 8, ...), so
    u_n = 1.  Then h_n = silu(g_n) * 1."""
    assert len(targets) == 32
    E, H, I = 1, 32, 32
    gate = np.full((E, I, 1, 32), 8, np.uint8)
    up = np.full((E, I, 1, 32), 8, np.uint8)
    for n, g in enumerate(targets):
        b = (g + 8) // 16
        c = g - 16 * b
        assert -8 <= b <= 7 and -8 <= c <= 7, g
        gate[0, n, 0, 1] = 8 + b
        gate[0, n, 0, 2] = 8 + c
        up[0, n, 0, 2] = 9
    pack = lambda codes: (codes[..., :16] | (codes[..., 16:] << 4)).astype(np.uint8)
    one = np.full((E, I, 1), 0x3C00, np.uint16)          # fp16 1.0
    down_q = np.full((E, H, 1, 16), 0x88, np.uint8)
    down_d = np.full((E, H, 1), 0x3C00, np.uint16)
    router = np.ones((E, H), np.float32)
    L = orc.MoE(router, pack(gate), one, pack(up), one.copy(), down_q, down_d, 1)
    x = np.zeros((1, H), np.float32)
    x[0, :3] = (127.0, 16.0, 1.0)
    return L, x


def test_silu_through_gate_up(orc):
    L, x = _silu_layer(orc, SILU_G)
    xq, xds = orc.quantize_q8_1(x)
    assert xq[0, :3].tolist() == [127, 16, 1] and orc.f16_to_f32(xds[0, 0, :1])[0] == 1.0
    h = L.gate_up(x, np.zeros((1, 1), np.int32))[0]
    g = np.array(SILU_G, np.float64)
    # the curve: h = g * sigma(g) with scipy's logistic function, to one fp32 ulp
    want = (g * expit(g)).astype(np.float32)
    assert (np.abs(h.astype(np.float64) - want) <= np.spacing(np.abs(want))).all()
    # silu(0) = 0
    assert h[SILU_G.index(0)] == 0.0
    # large positive g: silu(g) = g (1 - e^-g) rounds to g itself in fp32
    for gv in (20, 30, 40, 50, 60, 88, 100, 119):
        assert h[SILU_G.index(gv)] == np.float32(gv)
    # large negative g: silu(g) = g e^g / (1 + e^g), negative and vanishing
    for gv, bound in ((-20, 1e-7), (-40, 1e-15), (-60, 1e-24), (-100, 1e-40)):
        hv = float(h[SILU_G.index(gv)])
        assert -bound < hv <= 0.0, (gv, hv)
    assert float(h[SILU_G.index(-119)]) <= 0.0
    # the sign of the curve: silu(g) > 0 for g > 0, silu(g) < 0 for g < 0 (finite tail)
    for gv in (1, 2, 3, 5, 8, 10, 17):
        assert h[SILU_G.index(gv)] > 0 and h[SILU_G.index(-gv)] < 0
    # silu(g) - silu(-g) = g (sigma(g) + sigma(-g)) = g
    for gv in (1, 2, 3, 5, 8, 10, 17, 20, 30):
        d = float(h[SILU_G.index(gv)]) - float(h[SILU_G.index(-gv)])
        assert abs(d - gv) <= 4 * np.spacing(np.float32(gv)), (gv, d)
    # the minimum of silu lies near g = -1.28 at about -0.2785: the values at
    # -1 and -2 sit above it and below zero
    assert -0.2785 < h[SILU_G.index(-1)] < -0.26 and -0.2785 < h[SILU_G.index(-2)] < -0.23


def test_admissibility_check_rejects_a_wrong_routing(orc):
    # the rule the GPU decode tests apply to rows whose ids differ from the
    # float64 top-k: the exact top-k passes, a swap of two near-equal logits
    # passes, a swap that is not a near tie fails, and duplicates fail
    from tests._util import check_ids_admissible
    rng = np.random.default_rng(18)
    E, H, k = 32, 256, 4
    R = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    X = rng.standard_normal((2, H)).astype(np.float32)
    lg = orc.router_logits(R, X)
    ids = orc.topk(lg.astype(np.float32), k)
    _, differ = check_ids_admissible(orc, R, X, ids, k)
    assert differ == []
    # plant a near tie: router row of the 5th-ranked expert := the 4th's
    order = np.argsort(-lg[0], kind="stable")
    R2 = R.copy()
    R2[order[4]] = R2[order[3]]
    lg2 = orc.router_logits(R2, X)
    ids2 = orc.topk(lg2.astype(np.float32), k)
    swapped = ids2.copy()
    swapped[0, k - 1] = max(order[3], order[4])   # the higher index: lg2 equal
    _, differ = check_ids_admissible(orc, R2, X, swapped, k)
    assert differ == [0]
    wrong = ids.copy()
    wrong[0, k - 1] = order[E - 1]                 # the smallest logit of the row
    with pytest.raises(AssertionError):
        check_ids_admissible(orc, R, X, wrong, k)
    dup = ids.copy()
    dup[1, 1] = dup[1, 0]
    with pytest.raises(AssertionError):
        check_ids_admissible(orc, R, X, dup, k)
