"""GPU parity of gemv_bf16, quantize_q8_1 and gemv_q4_0 against the oracle,
through the C ABI (moe_matvec_amd binding)."""
import numpy as np
import pytest
import torch

import synth
from tests._util import np16, npc, rel_l2_rows

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-3   # rel-L2 per output row for BF16 GEMV
Q4_TOL = 2e-3     # rel-L2 per output row for Q4_0 x Q8_1 GEMV (vs the W4A8 result)
# what the W4A8 arithmetic keeps: exact int32 block dots, then fp32 scale
# products and sums (rel-L2 <= 2e-7 measured against the float64 oracle)
Q4_ARITH_TOL = 1e-5


# ---------------------------------------------------------------------------
# BF16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,B", [
    (1024, 1024, 1),      # the 1024 x 1024 correctness case (seed 0)
    (1000, 1016, 3),      # ragged rows and a ragged chunk tail
    (37, 72, 8),
    (4097, 2560, 2),
    (2560, 9728, 1),
    (513, 8, 5),
    (9, 4096, 8),
    (1, 512, 1),          # a single output row
    (1, 8, 8),            # a single row of the smallest K
])
def test_bf16_parity(mm, orc, dev, N, K, B):
    W = synth.bf16_weights(N, K, 0, "bf16", N, K, device=dev)
    X = synth.activations(B, K, 0, "bf16", N, K, device=dev)
    y = mm.gemv_bf16(W, X)
    torch.cuda.synchronize()
    ref = orc.gemv_bf16(np16(W), npc(X))
    assert rel_l2_rows(npc(y), ref) <= BF16_TOL


@pytest.mark.parametrize("N,K,B", [(777, 1032, 8), (777, 1032, 1), (300, 2560, 8), (35, 9728, 3)])
def test_bf16_integer_pin_bit_exact(mm, orc, dev, N, K, B):
    # small integers: every product and partial sum is exact in fp32 (and x
    # is exact in bf16, so its hi/lo split has lo = 0 on the B >= 2 path)
    g = torch.Generator().manual_seed(1)
    Wf = torch.randint(-8, 9, (N, K), generator=g).float()
    Xf = torch.randint(-16, 17, (B, K), generator=g).float()
    y = mm.gemv_bf16(Wf.to(torch.bfloat16).to(dev), Xf.to(dev))
    want = (Xf.double() @ Wf.double().T).numpy()
    assert np.array_equal(npc(y).astype(np.float64), want)


@pytest.mark.parametrize("N,K", [(2560, 2560), (19456, 2560), (2560, 9728)])
@pytest.mark.parametrize("B", [1, 8])
def test_bf16_full_size_decode_shapes(mm, orc, dev, N, K, B):
    # the dense decode set at full size (attn-out, fused gate+up, down), in
    # the configuration the benchmark times
    W = synth.bf16_weights(N, K, 0, "full", N, K, device=dev)
    X = synth.activations(B, K, 0, "full", N, K, B, device=dev)
    y = mm.gemv_bf16(W, X)
    torch.cuda.synchronize()
    assert rel_l2_rows(npc(y), orc.gemv_bf16(np16(W), npc(X))) <= BF16_TOL


def test_bf16_batch_invariance_and_determinism(mm, dev):
    # B >= 2 runs on the matrix cores with x split into bf16 hi + lo: column b
    # of the product depends on x row b alone, so every B >= 2 gives the same
    # bits for a row, and the B = 1 kernel (fp32 FMAs) agrees within rounding
    for N, K in ((3000, 2560), (700, 9728), (300, 1016), (129, 3072)):
        W = synth.bf16_weights(N, K, 0, "inv", K, device=dev)
        X = synth.activations(8, K, 0, "inv", K, device=dev)
        y8 = mm.gemv_bf16(W, X)
        assert torch.equal(y8, mm.gemv_bf16(W, X))
        for b in range(8):
            y1 = mm.gemv_bf16(W, X[b].clone())
            pair = mm.gemv_bf16(W, X[[b, (b + 3) % 8]].contiguous())[0]
            assert torch.equal(pair, y8[b])
            assert rel_l2_rows(npc(y1)[None], npc(y8[b])[None]) <= 1e-5
        for B in (3, 4, 5, 6, 7):
            assert torch.equal(mm.gemv_bf16(W, X[:B].contiguous()), y8[:B])


@pytest.mark.parametrize("knob", ["1168216", "1328216", "1168316", "1088208", "1164216"])
def test_bf16_lds_mfma_variants(mm, orc, dev, path, knob):
    # B >= 2, K % 512 == 0: the chunk loop instead of unrolled chunks, 32-row
    # workgroups, three chunks in flight and 8-row tiles give the default's
    # bits (a row's order depends on the waves per workgroup only); 4 waves
    # per workgroup sum the k-steps in another grouping: within rounding
    for N, K, B in ((1000, 2560, 8), (300, 2048, 5), (257, 4096, 3), (130, 9728, 8),
                    (90, 9728, 2), (17, 3072, 4), (1, 512, 2)):
        W = synth.bf16_weights(N, K, 0, "mlb", N, K, device=dev)
        X = synth.activations(B, K, 0, "mlb", N, K, device=dev)
        y0 = mm.gemv_bf16(W, X)
        path(BF16_ML=int(knob))
        y = mm.gemv_bf16(W, X)
        path(BF16_ML=0)
        if knob == "1164216":
            assert rel_l2_rows(npc(y), npc(y0)) <= 1e-6
            assert rel_l2_rows(npc(y), orc.gemv_bf16(np16(W), npc(X))) <= BF16_TOL
        else:
            assert torch.equal(y, y0)


@pytest.mark.parametrize("knobs", [dict(BF16_XL=-1, BF16_ROWS=1, BF16_WAVES=1),
                                   dict(BF16_XL=-1, BF16_ROWS=2, BF16_WAVES=4),
                                   dict(BF16_XL=-1, BF16_ROWS=4, BF16_WAVES=1),
                                   dict(BF16_XL=2), dict(BF16_XL=4), dict(BF16_XL=5),
                                   dict(BF16_XL=8), dict(BF16_XL=10), dict(BF16_XL=16)])
def test_bf16_b1_variants_identical(mm, dev, path, knobs):
    # every B = 1 variant (x from L1/L2 or staged in LDS, rows per wave, waves
    # per workgroup) sums each row in the same order: all give the same bits
    for N, K in ((1000, 2560), (2560, 9728), (333, 1016), (300, 2048), (257, 4096),
                 (100, 8192), (9000, 2560), (2561, 9728), (2555, 2560), (4097, 4096)):
        W = synth.bf16_weights(N, K, 0, "var", N, K, device=dev)
        x = synth.activations(1, K, 0, "var", N, K, device=dev)
        y0 = mm.gemv_bf16(W, x)
        path(**knobs)
        y1 = mm.gemv_bf16(W, x)
        path(**{k: 0 for k in knobs})
        assert torch.equal(y0, y1)


@pytest.mark.parametrize("ks", ["4", "8", "16"])
def test_bf16_mfma_split_variants(mm, orc, dev, path, ks):
    # the B >= 2 path with 4, 8 or 16 waves per 16-row tile
    N, K, B = 100, 1016, 5
    W = synth.bf16_weights(N, K, 0, "mfma", device=dev)
    X = synth.activations(B, K, 0, "mfma", device=dev)
    path(BF16_WAVES=int(ks))
    y = mm.gemv_bf16(W, X)
    path(BF16_WAVES=0)
    assert rel_l2_rows(npc(y), orc.gemv_bf16(np16(W), npc(X))) <= BF16_TOL


def test_bf16_leading_dimensions(mm, orc, dev):
    N, K = 300, 512
    Wp = synth.bf16_weights(N, K + 64, 0, "ld", device=dev)
    Xp = synth.activations(3, K + 8, 0, "ld", device=dev)
    W, X = Wp[:, :K], Xp[:, :K]
    out = torch.full((3, N + 5), 7.0, device=dev)
    mm.gemv_bf16(W, X, out=out[:, :N])
    ref = orc.gemv_bf16(np16(Wp), npc(Xp), K=K)
    assert rel_l2_rows(npc(out[:, :N]), ref) <= BF16_TOL
    assert (out[:, N:] == 7.0).all()


# ---------------------------------------------------------------------------
# Q8_1
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,K,scale", [(1, 4096, 1.0), (8, 2048, 1.0), (3, 96, 1e-3),
                                       (2, 32, 3e4), (5, 512, 1e-6)])
def test_quantize_q8_1_bit_exact(mm, orc, dev, B, K, scale):
    X = synth.activations(B, K, 0, "q8", B, K, device=dev) * scale
    X[0, :32] = 0.0                                  # an all-zero block
    if K >= 96:
        X[-1, 64:96] = 0.0
        X[-1, 70] = -2.5                             # a single-value block
    buf = mm.quantize_q8_1(X)
    torch.cuda.synchronize()
    q_ref, ds_ref = orc.quantize_q8_1(npc(X))
    codes, ds = mm.split_q8_1(buf, B, K)
    assert np.array_equal(npc(codes), q_ref)
    assert np.array_equal(np16(ds), ds_ref)


def test_quantize_q8_1_halfway_block_sums(mm, orc, dev):
    # blocks whose fp32 product d32 * sum q is an fp16 halfway point: s must be
    # the rounding of the fp32 product (a fused multiply-convert rounds once
    # and gives the other neighbour), in the standalone quantizer and in the
    # MoE path's staged Q8_1(x), which use the same routine
    from tests._util import q8_1_halfway_blocks
    X = torch.from_numpy(q8_1_halfway_blocks(orc, 64).reshape(8, 256)).to(dev)
    buf = mm.quantize_q8_1(X)
    torch.cuda.synchronize()
    q_ref, ds_ref = orc.quantize_q8_1(npc(X))
    codes, ds = mm.split_q8_1(buf, 8, 256)
    assert np.array_equal(npc(codes), q_ref)
    assert np.array_equal(np16(ds), ds_ref)


def test_quantize_q8_1_worked_example(mm, dev):
    from tests.test_oracle_q8_1 import _golden
    x, q, d, s = _golden()
    buf = mm.quantize_q8_1(torch.from_numpy(x)[None].to(dev))
    codes, ds = mm.split_q8_1(buf, 1, 32)
    assert np.array_equal(npc(codes)[0], q)
    assert np16(ds)[0, 0, 0] == d and np16(ds)[0, 0, 1] == s


# ---------------------------------------------------------------------------
# Q4_0
# ---------------------------------------------------------------------------

def _q4(mm, N, K, dev, *tags):
    qs, d = synth.q4_0_weights(N, K, 0, "q4", N, K, *tags, device=dev)
    return mm.Q4_0(qs, d), npc(qs), np16(d)


@pytest.mark.parametrize("N,K,B", [
    (4096, 4096, 1), (1100, 4096, 8), (2048, 512, 1), (515, 512, 8),
    (333, 2048, 3), (77, 96, 2), (64, 32, 1), (130, 1024, 6), (700, 8192, 2),
    (1, 32, 1), (1, 4096, 8), (200, 4096, 4), (300, 4096, 5),
])
def test_q4_0_parity(mm, orc, dev, N, K, B):
    W, qs, d = _q4(mm, N, K, dev)
    X = synth.activations(B, K, 0, "q4x", N, K, device=dev)
    y_x = mm.gemv_q4_0(W, x=X)
    xq = mm.quantize_q8_1(X)
    y_q = mm.gemv_q4_0(W, xq=xq, B=B)
    torch.cuda.synchronize()
    # on-the-fly quantization inside the GEMV equals quantize_q8_1 + Xq bit for
    # bit where both take the same kernel (the matrix cores from B = 3 for x,
    # from B = 5 for xq, at K <= 4096), within rounding otherwise
    if K > 4096 or B <= 2 or B >= 5:
        assert torch.equal(y_x, y_q)
    else:
        assert rel_l2_rows(npc(y_x), npc(y_q).astype(np.float64)) <= Q4_ARITH_TOL
    # x and xq together: x is quantized into xq, then xq is read
    buf = torch.full_like(xq, 0x5A)
    y_b = mm.gemv_q4_0(W, x=X, xq=buf)
    assert torch.equal(buf, xq) and torch.equal(y_b, y_q)
    q_ref, ds_ref = orc.quantize_q8_1(npc(X))
    ref = orc.gemv_q4_0(qs, d, q_ref, ds_ref)
    assert rel_l2_rows(npc(y_x), ref) <= Q4_TOL


@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096)])
@pytest.mark.parametrize("B", [1, 8])
def test_q4_0_full_size(mm, orc, dev, N, K, B):
    # the Q4_0 decode shapes at full size; B = 8 as the benchmark runs it
    # (quantize into a buffer, then the product)
    W, qs, d = _q4(mm, N, K, dev, "full")
    X = synth.activations(B, K, 0, "q4full", N, K, B, device=dev)
    xq = torch.empty(mm.q8_1_bytes(K, B), dtype=torch.uint8, device=dev) if B > 1 else None
    y = mm.gemv_q4_0(W, x=X, xq=xq)
    torch.cuda.synchronize()
    xq_ref, xds_ref = orc.quantize_q8_1(npc(X))
    ref = orc.gemv_q4_0(qs, d, xq_ref, xds_ref)
    assert rel_l2_rows(npc(y), ref) <= Q4_TOL


def test_q4_0_unit_scale_pin_bit_exact(mm, dev):
    g = torch.Generator().manual_seed(2)
    N, K, B = 700, 2048, 8
    codes = torch.randint(0, 16, (N, K // 32, 32), generator=g, dtype=torch.uint8)
    qs = (codes[..., :16] | (codes[..., 16:] << 4)).contiguous()
    d = torch.ones((N, K // 32), dtype=torch.float16)
    # x integer-valued with a +-127 in every block: Q8_1 gives d = 1, q = x
    x = torch.randint(-127, 128, (B, K), generator=g).float()
    x.view(B, -1, 32)[:, :, 3] = 127.0
    W = mm.Q4_0(qs.to(dev), d.to(dev))
    y = mm.gemv_q4_0(W, x=x.to(dev))
    want = x.double() @ (codes.reshape(N, K).double() - 8).T
    assert np.array_equal(npc(y).astype(np.float64), want.numpy())


def test_q4_0_batch_invariance(mm, dev):
    # each row of a B-row call against the same row in other calls: bit for
    # bit within one kernel (the dot4 kernels: K > 4096 or B <= 2 with fp32 x;
    # the matrix cores: B >= 3 at K <= 4096), within rounding across the two
    for N, K in ((1500, 4096), (700, 8192), (129, 2560)):
        W, _, _ = _q4(mm, N, K, dev, "inv")
        Bmax = min(8, mm.Q4_MAX_XK // K)
        X = synth.activations(Bmax, K, 0, "q4inv", K, device=dev)
        y8 = mm.gemv_q4_0(W, x=X)
        assert torch.equal(y8, mm.gemv_q4_0(W, x=X))
        for b in range(Bmax):
            y1 = mm.gemv_q4_0(W, x=X[b:b + 1].clone())
            if K > 4096:
                assert torch.equal(y1, y8[b:b + 1])
                continue
            y3 = mm.gemv_q4_0(W, x=X[[b, (b + 1) % Bmax, (b + 2) % Bmax]].clone())
            assert torch.equal(y8[b], y3[0])
            assert torch.equal(y1[0], mm.gemv_q4_0(W, x=X[[b, b]].clone())[1])
            assert rel_l2_rows(npc(y8[b]), npc(y1[0]).astype(np.float64)) <= Q4_ARITH_TOL


@pytest.mark.parametrize("N,K", [(4096, 4096), (20000, 4096), (1000, 96), (777, 2560),
                                 (33, 3840), (16, 512), (1, 128), (17, 32)])
def test_q4_0_both_kernels_every_b(mm, orc, dev, path, N, K):
    # the matrix-core kernel forced from B = 1 and the dot4 kernels forced at
    # every B, from fp32 x and from a Q8_1 buffer (the same rows bit for bit),
    # against the oracle on the same Q8_1 codes (20000 rows: several tiles per
    # workgroup on any GPU of up to 1250 compute units)
    W, qs, d = _q4(mm, N, K, dev, "both")
    for B in range(1, 9):
        X = synth.activations(B, K, 0, "q4both", N, K, B, device=dev)
        q_ref, ds_ref = orc.quantize_q8_1(npc(X))
        ref = orc.gemv_q4_0(qs, d, q_ref, ds_ref)
        for sw in (1, -1):
            path(Q4_MF=sw)
            y = mm.gemv_q4_0(W, x=X)
            y_q = mm.gemv_q4_0(W, xq=mm.quantize_q8_1(X), B=B)
            torch.cuda.synchronize()
            assert torch.equal(y, y_q), (B, sw)
            assert rel_l2_rows(npc(y), ref) <= Q4_ARITH_TOL, (B, sw)


@pytest.mark.parametrize("N,K", [(1000, 11008), (257, 9728), (300, 14336), (33, 16352),
                                 (129, 2560), (65, 3840), (70, 6144), (200, 2080)])
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_q4_0_ragged_rows_equal_grid_stride(mm, orc, dev, path, N, K, B):
    # rows of 64 < K/32 <= 512 blocks that are not whole 64-block steps (the
    # down projections of the 7B-9B models among them) take the whole-row
    # kernel with a ragged last step at B <= 4: the same rows, bit for bit, as
    # the grid-stride kernel, from fp32 x and from a Q8_1 buffer, and the
    # oracle's on the same codes; the rows of 16352 end one block short of
    # eight 64-block steps, those of 2080 one block into the second (the int8
    # matrix cores, which take K <= 4096 from
    # B = 3, are held off: their sums run in another order)
    if B * K > mm.Q4_MAX_XK:
        pytest.skip("B * K above the staging limit")
    path(Q4_MF=-1)
    W, qs, d = _q4(mm, N, K, dev, "ragged")
    X = synth.activations(B, K, 0, "q4ragged", N, K, device=dev)
    xq = mm.quantize_q8_1(X)
    y = mm.gemv_q4_0(W, x=X)
    y_q = mm.gemv_q4_0(W, xq=xq, B=B)
    path(Q4_GENERIC=1)
    y_g = mm.gemv_q4_0(W, x=X)
    torch.cuda.synchronize()
    assert torch.equal(y, y_q) and torch.equal(y, y_g)
    q_ref, ds_ref = orc.quantize_q8_1(npc(X))
    assert rel_l2_rows(npc(y), orc.gemv_q4_0(qs, d, q_ref, ds_ref)) <= Q4_ARITH_TOL


@pytest.mark.parametrize("N,K,B", [(1, 4096, 1), (17, 8192, 1), (33, 4096, 2), (5, 11008, 1),
                                   (3, 8192, 4)])
def test_q4_0_fewer_rows_than_a_workgroup(mm, orc, dev, N, K, B):
    # 8-wave workgroups own 16 rows: with fewer, the missing rows repeat the
    # last one in bounds and store nothing; x and a Q8_1 buffer agree
    W, qs, d = _q4(mm, N, K, dev, "few")
    X = synth.activations(B, K, 0, "q4few", N, K, B, device=dev)
    y = mm.gemv_q4_0(W, x=X)
    y_q = mm.gemv_q4_0(W, xq=mm.quantize_q8_1(X), B=B)
    torch.cuda.synchronize()
    q_ref, ds_ref = orc.quantize_q8_1(npc(X))
    ref = orc.gemv_q4_0(qs, d, q_ref, ds_ref)
    assert y.shape == (B, N)
    assert rel_l2_rows(npc(y), ref) <= Q4_ARITH_TOL
    assert rel_l2_rows(npc(y_q), ref) <= Q4_ARITH_TOL


@pytest.mark.parametrize("B", [2, 3, 5, 7])
def test_q4_0_strided_x_and_y(mm, orc, dev, B):
    # x rows with ldx > K at an offset, y rows with ldy > N (the padding must
    # stay untouched), from fp32 x and from a Q8_1 buffer: the dot4 kernels
    # (B = 2; B = 3, 5 from the buffer) and the matrix cores (B = 3, 5, 7
    # from x; B = 7 from the buffer)
    N, K = 1200, 1024
    W, qs, d = _q4(mm, N, K, dev, "stride")
    Xb = synth.activations(B, K + 64, 0, "q4s", B, device=dev)
    X = Xb[:, 32:32 + K]
    q_ref, ds_ref = orc.quantize_q8_1(npc(X))
    ref = orc.gemv_q4_0(qs, d, q_ref, ds_ref)
    for use_xq in (False, True):
        Yb = torch.full((B, N + 7), 123.0, device=dev)
        if use_xq:
            mm.gemv_q4_0(W, xq=mm.quantize_q8_1(X), B=B, out=Yb[:, :N])
        else:
            mm.gemv_q4_0(W, x=X, out=Yb[:, :N])
        torch.cuda.synchronize()
        assert rel_l2_rows(npc(Yb[:, :N]), ref) <= Q4_ARITH_TOL
        assert torch.all(Yb[:, N:] == 123.0)


@pytest.mark.parametrize("env", [
    dict(Q4_RP=2), dict(Q4_RP=4), dict(Q4_RP=6), dict(Q4_RP=8),
    dict(Q4_GENERIC=1, Q4_WG_PER_CU=1),
    dict(Q4_GENERIC=1, Q4_WG_PER_CU=3),
    dict(Q4_GENERIC=1, Q4_WG_PER_CU=16),
])
def test_q4_0_grid_variants_identical(mm, dev, path, env):
    # rows per workgroup, the whole-row kernel versus the grid-stride one:
    # no row's sums change (the dot4 kernels at every B)
    path(Q4_MF=-1)
    for N, K, B in ((4096, 4096, 1), (1100, 512, 8), (515, 2048, 3), (300, 8192, 2),
                    (2000, 1024, 1)):
        W, _, _ = _q4(mm, N, K, dev, "grid")
        X = synth.activations(B, K, 0, "q4grid", N, device=dev)
        y0 = mm.gemv_q4_0(W, x=X)
        path(**env)
        y1 = mm.gemv_q4_0(W, x=X)
        y2 = mm.gemv_q4_0(W, xq=mm.quantize_q8_1(X), B=B)
        path(**{k: 0 for k in env})
        assert torch.equal(y0, y1) and torch.equal(y0, y2)
