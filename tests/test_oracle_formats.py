"""Pins of the oracle's number-format conversions against independent
implementations (numpy's float16 cast, torch's bfloat16 cast) and closed forms."""
import os

import numpy as np
import torch


def test_f16_roundtrip_every_value(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(f[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(f[nan]).all()
    back = orc.f32_to_f16(f[~nan])
    assert np.array_equal(back, h[~nan])


def test_f16_halfway_cases_round_to_even(orc):
    # midpoints between consecutive fp16 values (normal and subnormal ranges)
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)          # exact in fp32
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    got = orc.f32_to_f16(np.concatenate([mid, -mid]))
    want = np.concatenate([mid, -mid]).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    # and the rule itself: ties go to the even code
    even = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(got[: len(h)], even)


def test_f16_random_and_extremes(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(100000) * 1e-6).astype(np.float32),   # subnormal fp16 range
        (rng.standard_normal(100000) * 3e4).astype(np.float32),    # near overflow
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 2.0 ** -24, 1e-40, np.inf, -np.inf], np.float32),
    ])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f32_to_f16(x), want)


def test_bf16_against_torch(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # halfway cases: low 16 bits exactly 0x8000
    half = ((rng.integers(0, 2 ** 16, 20000, dtype=np.uint64).astype(np.uint32) << 16)
            | np.uint32(0x8000)).view(np.float32)
    half = half[np.isfinite(half)]
    x = np.concatenate([x, half, np.float32([0.0, -0.0, 1.0, -1.0])])
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16(x), want)
    # widening is exact: bf16 bits << 16
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = orc.bf16_to_f32(h)
    assert np.array_equal(f.view(np.uint32), h.astype(np.uint32) << 16)


# ---------------------------------------------------------------------------
# interchange blocks: the 36-byte Q8_1 and 18-byte Q4_0 blocks the pages name,
# converted to and from the library's planar layout (test utilities)
# ---------------------------------------------------------------------------

def test_q8_1_interchange_block_golden(orc):
    from tests._util import q8_1_from_blocks, q8_1_to_blocks, read_golden_blocks
    from tests.test_oracle_q8_1 import _golden
    g = read_golden_blocks(os.path.join(os.path.dirname(__file__), "golden",
                                        "interchange_blocks.txt"))
    blk = g["q8_1"].reshape(1, 1, 36)
    x, q, d, s = _golden()
    codes, ds = q8_1_from_blocks(blk)
    assert np.array_equal(codes[0], q) and ds[0, 0, 0] == d and ds[0, 0, 1] == s
    oq, ods = orc.quantize_q8_1(x[None])
    assert np.array_equal(q8_1_to_blocks(oq, ods), blk)


def test_q4_0_interchange_block_golden():
    from tests._util import q4_0_from_blocks, q4_0_to_blocks, read_golden_blocks
    from tests.test_oracle_gemv import _dense_q4
    g = read_golden_blocks(os.path.join(os.path.dirname(__file__), "golden",
                                        "interchange_blocks.txt"))
    blk = g["q4_0"].reshape(1, 1, 18)
    qs, d = q4_0_from_blocks(blk)
    w = _dense_q4(qs, d)[0]
    assert np.array_equal(w, np.array([(i % 16) - 8 for i in range(32)], np.float64))
    assert np.array_equal(q4_0_to_blocks(qs, d), blk)


def test_interchange_round_trips():
    from tests._util import q4_0_from_blocks, q4_0_to_blocks, q8_1_from_blocks, q8_1_to_blocks
    rng = np.random.default_rng(21)
    codes = rng.integers(-127, 128, (3, 96)).astype(np.int8)
    ds = rng.integers(0, 1 << 16, (3, 3, 2)).astype(np.uint16)
    c2, d2 = q8_1_from_blocks(q8_1_to_blocks(codes, ds))
    assert np.array_equal(c2, codes) and np.array_equal(d2, ds)
    assert q8_1_to_blocks(codes, ds).nbytes == codes.nbytes + ds.nbytes   # same bytes
    qs = rng.integers(0, 256, (5, 4, 16)).astype(np.uint8)
    d = rng.integers(0, 1 << 16, (5, 4)).astype(np.uint16)
    q2, e2 = q4_0_from_blocks(q4_0_to_blocks(qs, d))
    assert np.array_equal(q2, qs) and np.array_equal(e2, d)
