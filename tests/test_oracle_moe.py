"""Pins of the oracle's router, top-k, gate weights, gather lists and whole MoE
layer: numpy matmuls, a stable sort on (-value, index), Python's sorted(),
closed forms, and a dense numpy restatement of the layer on small cases."""
import numpy as np
import pytest

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
    silu = lambda z: z / (1 + np.exp(-z))
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
