"""Pins of the oracle's W4A16 product (Q4_0 weights x fp32 activations) and
row argmax, against independent numpy restatements, exact integer cases and
the already-pinned W4A8 product and top-k."""
import numpy as np
import pytest


def _codes(qs):
    """Independent unpacking of split-nibble blocks: [N, nb, 16] -> [N, nb*32]."""
    lo = (qs & 0x0F).astype(np.int64)
    hi = (qs >> 4).astype(np.int64)
    return np.concatenate([lo, hi], axis=2).reshape(qs.shape[0], -1)


def _random_q4(rng, N, K):
    qs = rng.integers(0, 256, size=(N, K // 32, 16), dtype=np.uint8)
    d = (rng.uniform(0.001, 0.05, size=(N, K // 32))).astype(np.float16).view(np.uint16)
    return qs, d


@pytest.mark.parametrize("N,K,B", [(1, 32, 1), (9, 96, 3), (40, 256, 8)])
def test_w4a16_matches_numpy_dequantized(orc, N, K, B):
    rng = np.random.default_rng(N * 7 + K)
    qs, d = _random_q4(rng, N, K)
    X = rng.standard_normal((B, K)).astype(np.float32)
    scale = np.repeat(d.view(np.float16).astype(np.float64), 32, axis=1)
    Wd = (_codes(qs) - 8).astype(np.float64) * scale
    np.testing.assert_allclose(orc.gemv_q4_0_f32(qs, d, X), X.astype(np.float64) @ Wd.T,
                               rtol=1e-12, atol=1e-14)


def test_w4a16_one_hot_selects_a_weight(orc):
    rng = np.random.default_rng(3)
    N, K = 17, 128
    qs, d = _random_q4(rng, N, K)
    codes = _codes(qs)
    for k in (0, 15, 16, 31, 32, 77, 127):   # both nibbles of a byte, several blocks
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        want = (codes[:, k] - 8) * d.view(np.float16)[:, k // 32].astype(np.float64)
        assert np.array_equal(orc.gemv_q4_0_f32(qs, d, x)[0], want)


def test_w4a16_equals_w4a8_when_q8_1_is_exact(orc):
    # integer x in [-127, 127] with a 127 in every block: Q8_1 has d = 1 and
    # codes = x, so the (pinned) W4A8 product and W4A16 agree exactly
    rng = np.random.default_rng(9)
    N, K, B = 23, 192, 4
    qs, d = _random_q4(rng, N, K)
    X = rng.integers(-127, 128, size=(B, K)).astype(np.float32)
    X.reshape(B, -1, 32)[:, :, 5] = 127.0
    xq, xds = orc.quantize_q8_1(X)
    assert np.array_equal(xq.astype(np.float32), X)
    assert np.array_equal(orc.gemv_q4_0_f32(qs, d, X), orc.gemv_q4_0(qs, d, xq, xds))


def test_argmax_matches_numpy_and_topk1(orc):
    rng = np.random.default_rng(11)
    for N in (1, 2, 63, 1000):
        Y = rng.standard_normal((5, N)).astype(np.float32)
        Y[1] = np.round(Y[1] * 2) / 2        # many exact ties
        ids = orc.argmax(Y)
        assert np.array_equal(ids, np.argmax(Y, axis=1))   # first occurrence of the max
        assert np.array_equal(ids, orc.topk(Y, 1)[:, 0])


def test_argmax_ties_and_signed_zero(orc):
    Y = np.zeros((4, 9), np.float32)
    Y[1, 3] = -0.0
    Y[1, 0] = -1.0                           # max is 0: indices 1.. tie, lowest wins
    Y[2, :] = -0.0
    Y[2, 6] = 0.0                            # -0 == +0: index 0 wins
    Y[3, 7] = 5.0
    Y[3, 8] = 5.0
    assert np.array_equal(orc.argmax(Y), [0, 1, 0, 7])
