"""Pins of the oracle's BF16 and Q4_0 x Q8_1 products against numpy float64
matmuls, integer matmuls and exact special cases."""
import numpy as np
import pytest


def _bf16_widen(Wb):
    """Independent widening: bf16 bits to fp32 by a 16-bit shift (numpy)."""
    return (Wb.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("N,K,B", [(1, 8, 1), (7, 40, 3), (64, 64, 8), (33, 256, 2)])
def test_bf16_matches_numpy(orc, N, K, B):
    rng = np.random.default_rng(N * 1000 + K)
    W = orc.f32_to_bf16((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    X = rng.standard_normal((B, K)).astype(np.float32)
    want = X.astype(np.float64) @ _bf16_widen(W).astype(np.float64).T
    got = orc.gemv_bf16(W, X)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_bf16_integer_exact_and_special(orc):
    rng = np.random.default_rng(5)
    N, K = 24, 64
    Wf = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    W = orc.f32_to_bf16(Wf)
    X = rng.integers(-20, 21, size=(2, K)).astype(np.float32)
    assert np.array_equal(orc.gemv_bf16(W, X), X.astype(np.int64) @ Wf.astype(np.int64).T)
    # one-hot x selects a column
    e = np.zeros((1, K), np.float32)
    e[0, 17] = 1.0
    assert np.array_equal(orc.gemv_bf16(W, e)[0], Wf[:, 17])
    # identity matrix returns x (values exactly representable)
    I = orc.f32_to_bf16(np.eye(K, dtype=np.float32))
    x = orc.bf16_to_f32(orc.f32_to_bf16(rng.standard_normal((1, K)).astype(np.float32)))
    assert np.array_equal(orc.gemv_bf16(I, x)[0], x[0].astype(np.float64))
    # leading dimension: a padded matrix gives the same result
    Wp = np.zeros((N, K + 8), np.uint16)
    Wp[:, :K] = W
    assert np.array_equal(orc.gemv_bf16(Wp, X, K=K), orc.gemv_bf16(W, X))


def _pack_q4(codes):
    """codes uint8 [N, nb, 32] (0..15) -> split-nibble qs [N, nb, 16]."""
    return (codes[..., :16] | (codes[..., 16:] << 4)).astype(np.uint8)


def _dense_q4(qs, d):
    """Independent dense decode of a planar Q4_0 matrix (numpy)."""
    lo = (qs & 0x0F).astype(np.int64)
    hi = (qs >> 4).astype(np.int64)
    codes = np.concatenate([lo, hi], axis=-1)           # [N, nb, 32]
    w = (codes - 8) * d.view(np.float16).astype(np.float64)[..., None]
    return w.reshape(qs.shape[0], -1)


def _q8_dense(q, ds):
    d = ds[..., 0].view(np.float16).astype(np.float64)
    return (q.reshape(q.shape[0], -1, 32) * d[..., None]).reshape(q.shape[0], -1)


def test_q4_unit_scale_integer_pin(orc):
    rng = np.random.default_rng(6)
    N, K, B = 37, 32 * 9, 3
    codes = rng.integers(0, 16, size=(N, K // 32, 32)).astype(np.uint8)
    qs = _pack_q4(codes)
    dw = np.full((N, K // 32), 0x3C00, np.uint16)           # fp16 1.0
    xq = rng.integers(-127, 128, size=(B, K)).astype(np.int8)
    xds = np.zeros((B, K // 32, 2), np.uint16)
    xds[..., 0] = 0x3C00
    Wint = codes.reshape(N, K).astype(np.int64) - 8
    want = xq.astype(np.int64) @ Wint.T
    assert np.array_equal(orc.gemv_q4_0(qs, dw, xq, xds), want)
    sums = orc.q4_0_block_sums(qs, xq)
    assert np.array_equal(sums.sum(-1), want)
    assert np.array_equal(sums[1, 4, 2], (Wint[4, 64:96] * xq[1, 64:96]).sum())


def test_q4_split_nibble_order(orc):
    # code[i] = (i*7 + 3) % 16 for i in 0..31; one-hot x at position p gives code[p] - 8
    codes = ((np.arange(32) * 7 + 3) % 16).astype(np.uint8)[None, None, :]
    qs = _pack_q4(codes)
    assert qs[0, 0, 0] == (codes[0, 0, 0] | (codes[0, 0, 16] << 4))
    dw = np.full((1, 1), 0x3C00, np.uint16)
    xq = np.eye(32, dtype=np.int8)
    xds = np.zeros((32, 1, 2), np.uint16)
    xds[..., 0] = 0x3C00
    got = orc.gemv_q4_0(qs, dw, xq, xds)[:, 0]
    assert np.array_equal(got, codes[0, 0].astype(np.int64) - 8)


def test_q4_power_of_two_scales_exact(orc):
    rng = np.random.default_rng(7)
    N, K, B = 9, 32 * 5, 2
    codes = rng.integers(0, 16, size=(N, K // 32, 32)).astype(np.uint8)
    qs = _pack_q4(codes)
    ew = rng.integers(-8, 4, size=(N, K // 32))
    dw = (2.0 ** ew).astype(np.float16).view(np.uint16)
    ex = rng.integers(-6, 2, size=(B, K // 32))
    xq = rng.integers(-127, 128, size=(B, K)).astype(np.int8)
    xds = np.zeros((B, K // 32, 2), np.uint16)
    xds[..., 0] = (2.0 ** ex).astype(np.float16).view(np.uint16)
    want = _q8_dense(xq, xds) @ _dense_q4(qs, dw).T          # all terms exact in float64
    assert np.array_equal(orc.gemv_q4_0(qs, dw, xq, xds), want)


def test_q4_random_matches_dense_decode(orc):
    rng = np.random.default_rng(8)
    N, K, B = 50, 32 * 12, 4
    codes = rng.integers(0, 16, size=(N, K // 32, 32)).astype(np.uint8)
    qs = _pack_q4(codes)
    dw = (rng.random((N, K // 32)) * 0.01 + 1e-4).astype(np.float16).view(np.uint16)
    x = rng.standard_normal((B, K)).astype(np.float32)
    xq, xds = orc.quantize_q8_1(x)
    want = _q8_dense(xq, xds) @ _dense_q4(qs, dw).T
    np.testing.assert_allclose(orc.gemv_q4_0(qs, dw, xq, xds), want, rtol=1e-12, atol=1e-14)
