"""Pins of the oracle's Q8_1 quantizer: a hand-derived worked example, exact
integer cases, zero and single-value blocks, the unrepresentable-scale rule
and the round-trip error bound."""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8_1_worked_example.txt")


def _golden():
    xs, qs, d, s = [], [], None, None
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] == "x":
            xs.append(float(parts[1]))
            qs.append(int(parts[2]))
        elif parts[0] == "d":
            d = int(parts[1], 16)
        elif parts[0] == "s":
            s = int(parts[1], 16)
    return np.array(xs, np.float32), np.array(qs, np.int8), d, s


def test_worked_example(orc):
    x, q, d, s = _golden()
    assert x.size == 32
    got_q, got_ds = orc.quantize_q8_1(x[None, :])
    assert np.array_equal(got_q[0], q)
    assert got_ds[0, 0, 0] == d and got_ds[0, 0, 1] == s


def test_integer_blocks_are_exact(orc):
    rng = np.random.default_rng(2)
    B, K = 3, 32 * 40
    x = rng.integers(-127, 128, size=(B, K)).astype(np.float32)
    blocks = x.reshape(B, -1, 32)
    # force a +-127 in every block so amax = 127 and d = 1 exactly
    blocks[:, :, 5] = np.where(rng.random(blocks.shape[:2]) < 0.5, 127, -127)
    x = blocks.reshape(B, K)
    q, ds = orc.quantize_q8_1(x)
    assert np.array_equal(q, x.astype(np.int8))
    assert (ds[:, :, 0] == 0x3C00).all()                       # fp16 1.0
    sums = x.reshape(B, -1, 32).sum(-1)
    assert np.array_equal(ds[:, :, 1], sums.astype(np.float16).view(np.uint16))


def test_block_sum_rounds_through_fp16(orc):
    # sum q = 2049 is not representable in fp16: RNE gives 2048 (0x6800)
    x = np.zeros(32, np.float32)
    x[:16] = 127.0
    x[16] = 17.0           # 16*127 + 17 = 2049
    q, ds = orc.quantize_q8_1(x[None])
    assert int(q.sum()) == 2049
    assert ds[0, 0, 1] == 0x6800


def test_zero_and_single_value_blocks(orc):
    x = np.zeros((1, 96), np.float32)
    x[0, 40] = -3.25
    x[0, 64 + 31] = 1e-3
    q, ds = orc.quantize_q8_1(x)
    assert not q[0, :32].any() and (ds[0, 0] == 0).all()
    assert q[0, 40] == -127 and np.count_nonzero(q[0, 32:64]) == 1
    assert ds[0, 1, 0] == np.float16(np.float32(3.25) / np.float32(127)).view(np.uint16)
    assert q[0, 95] == 127 and ds[0, 2, 1] == np.float16(
        np.float32(np.float32(1e-3) / np.float32(127)) * np.float32(127)).view(np.uint16)


def test_unrepresentable_scale_gives_zero_block(orc):
    # amax/127 <= 2^-25 rounds to fp16 zero: the block is stored as zeros
    x = np.zeros((1, 64), np.float32)
    x[0, :32] = np.float32(127 * 2.0 ** -25)
    x[0, 32:] = np.float32(127 * 2.0 ** -24)          # smallest fp16 subnormal scale
    q, ds = orc.quantize_q8_1(x)
    assert not q[0, :32].any() and (ds[0, 0] == 0).all()
    assert (q[0, 32:] == 127).all() and ds[0, 1, 0] == 0x0001


@pytest.mark.parametrize("scale", [1.0, 1e-3, 40.0])
def test_roundtrip_bound(orc, scale):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4, 32 * 64)) * scale).astype(np.float32)
    q, ds = orc.quantize_q8_1(x)
    blocks = x.reshape(4, -1, 32).astype(np.float64)
    amax = np.abs(blocks).max(-1)
    d32 = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)
    d16 = ds[:, :, 0].view(np.float16).astype(np.float64)
    recon = d16[..., None] * q.reshape(4, -1, 32)
    bound = d32[..., None] / 2 + 127 * np.abs(d32 - d16)[..., None] + 4 * np.spacing(amax)[..., None]
    assert (np.abs(blocks - recon) <= bound).all()
    # codes use the full range: the amax element maps to +-127
    assert (np.abs(q.reshape(4, -1, 32)).max(-1) == 127).all()


def test_row_stride_is_respected(orc):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 100)).astype(np.float32)
    q1, d1 = orc.quantize_q8_1(x, K=64)
    q2, d2 = orc.quantize_q8_1(np.ascontiguousarray(x[:, :64]))
    assert np.array_equal(q1, q2) and np.array_equal(d1, d2)


def test_block_sum_rounds_the_fp32_product(orc):
    # s = fp16(d32 * sum q) with d32 * sum q an fp32 product: at blocks where
    # that product is an fp16 halfway point, s follows round-to-nearest-even
    # of the fp32 value, not the rounding of the exact product
    from tests._util import q8_1_halfway_blocks
    X = q8_1_halfway_blocks(orc, 8)
    q, ds = orc.quantize_q8_1(X.reshape(1, -1))
    S = q.reshape(8, 32).astype(np.int64).sum(1)
    d32 = (np.abs(X).max(1) / np.float32(127.0)).astype(np.float32)
    p32 = (d32 * S.astype(np.float32)).astype(np.float32)
    assert np.array_equal(ds[0, :, 1], p32.astype(np.float16).view(np.uint16))
    exact = d32.astype(np.float64) * S
    assert not np.array_equal(ds[0, :, 1], exact.astype(np.float16).view(np.uint16))
    assert np.array_equal(ds[0, :, 0], d32.astype(np.float16).view(np.uint16))
