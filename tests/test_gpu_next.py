"""GPU parity of the LM-head pieces (on-device argmax, the 248,320-row BF16
GEMV feeding it) and of the W4A16 Q4_0 GEMV, against the oracle, through
the C ABI."""
import numpy as np
import pytest
import torch

import synth
from tests._util import np16, npc, rel_l2_rows

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-3   # rel-L2 per output row, BF16 GEMV
Q4_TOL = 2e-3     # rel-L2 per output row, Q4_0 weight products
W4A16_ARITH_TOL = 1e-4  # rel-L2 per row, W4A16 against float64: what its arithmetic keeps

VOCAB, HID = 248320, 2560   # LM head of the 2560-wide model


# ---------------------------------------------------------------------------
# argmax_rows
# ---------------------------------------------------------------------------

def _argmax_check(mm, orc, Y: torch.Tensor, N=None):
    """Y fp32 [B, ldy] on the device; argmax over the first N columns."""
    N = Y.shape[1] if N is None else N
    ids, vals = mm.argmax_rows(Y[:, :N])
    torch.cuda.synchronize()
    Yh = npc(Y[:, :N])
    want = orc.argmax(Yh)
    assert np.array_equal(npc(ids), want)
    got_v = npc(vals)
    ref_v = Yh[np.arange(Yh.shape[0]), want]
    # the value returned is the element itself (a -0 maximum comes back as +0)
    assert np.array_equal(got_v, ref_v + np.float32(0.0))


@pytest.mark.parametrize("N,B", [
    (1, 1), (3, 2), (4095, 1), (4096, 3), (4097, 8), (50001, 5), (VOCAB, 1), (VOCAB, 8),
])
def test_argmax_random(mm, orc, dev, N, B):
    Y = synth.normal((B, N), 1.0, 0, "argmax", N, B, device=dev)
    _argmax_check(mm, orc, Y)


def test_argmax_ties_lowest_index(mm, orc, dev):
    # the maximum planted at several positions, in different slices of 4096
    N, B = 3 * 4096 + 17, 4
    Y = synth.normal((B, N), 1.0, 0, "ties", device=dev)
    spots = [[9000, 4100, N - 1], [N - 1, 12287], [5, 4095, 4096], [0, 1, 2]]
    for b, s in enumerate(spots):
        Y[b, s] = 7.5
    _argmax_check(mm, orc, Y)
    ids, _ = mm.argmax_rows(Y)
    assert npc(ids).tolist() == [min(s) for s in spots]


def test_argmax_signed_zero_and_negative_rows(mm, orc, dev):
    N = 9000
    Y = -1.0 - synth.normal((4, N), 1.0, 0, "neg", device=dev).abs()
    Y[0, 7] = -0.0          # -0 before +0: equal values, the lower index wins
    Y[0, 8000] = 0.0
    Y[1, 3] = 0.0           # +0 before -0
    Y[1, 6000] = -0.0
    Y[2].fill_(-0.0)        # all -0: index 0, value +0
    Y[3, N - 1] = -0.5      # every value negative: the largest at the tail
    _argmax_check(mm, orc, Y)
    ids, vals = mm.argmax_rows(Y)
    assert npc(ids).tolist() == [7, 3, 0, N - 1]
    assert npc(vals).tolist() == [0.0, 0.0, 0.0, -0.5]


def test_argmax_strided_rows_and_stale_workspace(mm, orc, dev):
    B, N, ld = 6, 20000, 20480
    Y = synth.normal((B, ld), 1.0, 0, "stride", device=dev)
    Y[:, N:] = 100.0        # beyond N: must not be seen
    ws = torch.full((mm.argmax_workspace_bytes(N, B),), 0xFF, dtype=torch.uint8, device=dev)
    ids, vals = mm.argmax_rows(Y[:, :N], workspace=ws)
    torch.cuda.synchronize()
    want = orc.argmax(npc(Y[:, :N]))
    assert np.array_equal(npc(ids), want)
    assert np.array_equal(npc(vals), npc(Y)[np.arange(B), want])


# ---------------------------------------------------------------------------
# LM head: BF16 GEMV over the vocabulary, then argmax on the device
# ---------------------------------------------------------------------------

def test_lm_head_gemv_argmax(mm, orc, dev):
    W = synth.bf16_weights(VOCAB, HID, 0, "lm_head", device=dev)
    for B in (1, 8):
        X = synth.activations(B, HID, 0, "lm_head", B, device=dev)
        y = mm.gemv_bf16(W, X)
        ids, vals = mm.argmax_rows(y)
        torch.cuda.synchronize()
        Yg = npc(y)
        ref = orc.gemv_bf16(np16(W), npc(X))
        assert rel_l2_rows(Yg, ref) <= BF16_TOL
        # the decision is taken on the fp32 logits the GEMV produced
        assert np.array_equal(npc(ids), orc.argmax(Yg))
        assert np.array_equal(npc(vals), Yg[np.arange(B), npc(ids)])
        # and it is the exact argmax unless the top two are within rounding
        top = np.argmax(ref, axis=1)
        gap = np.abs(ref[np.arange(B), top] - ref[np.arange(B), npc(ids)])
        assert np.all(gap <= 1e-4 * np.abs(ref).max(axis=1))


# ---------------------------------------------------------------------------
# W4A16: Q4_0 weights x fp32 activations
# ---------------------------------------------------------------------------

def _q4(mm, N, K, dev, *tags):
    qs, d = synth.q4_0_weights(N, K, 0, "w4a16", N, K, *tags, device=dev)
    return mm.Q4_0(qs, d), npc(qs), np16(d)


@pytest.mark.parametrize("N,K,B", [
    (4096, 4096, 1), (11008, 4096, 1), (4096, 4096, 4), (1000, 512, 8), (515, 1024, 3),
    (4097, 2048, 8), (300, 8192, 2), (9, 4096, 4), (1, 512, 1), (2560, 8192, 1),
    # the general kernel: more rows at K = 4096 (up to the 8 of a batch), any K % 32
    (11008, 4096, 8), (4096, 4096, 5), (9728, 2560, 8), (2560, 2560, 1), (1000, 96, 3),
    (333, 11008, 3), (700, 8192, 4), (65, 36864, 1), (2049, 32, 8), (17, 9728, 2),
])
def test_w4a16_parity(mm, orc, dev, N, K, B):
    W, qs, d = _q4(mm, N, K, dev)
    X = synth.activations(B, K, 0, "w4a16", N, K, device=dev)
    y = mm.gemv_q4_0_f32(W, X)
    torch.cuda.synchronize()
    ref = orc.gemv_q4_0_f32(qs, d, npc(X))
    assert rel_l2_rows(npc(y), ref) <= Q4_TOL


@pytest.mark.parametrize("N,K,B", [(777, 2048, 8), (300, 2560, 8), (129, 4096, 8),
                                   (65, 11008, 3)])
def test_w4a16_integer_pin_bit_exact(mm, orc, dev, N, K, B):
    # power-of-two scales and integer activations: every partial sum is an
    # exact fp32 value, so the product must match the float64 oracle exactly
    # (the whole-row kernel at 2048 x 8, the general one otherwise)
    g = torch.Generator().manual_seed(3)
    qs = torch.randint(0, 256, (N, K // 32, 16), generator=g, dtype=torch.uint8)
    scales = torch.tensor([1.0, 0.5, 2.0, 0.25], dtype=torch.float16)
    d = scales[torch.randint(0, 4, (N, K // 32), generator=g)]
    X = torch.randint(-16, 17, (B, K), generator=g).float()
    y = mm.gemv_q4_0_f32(mm.Q4_0(qs.to(dev), d.to(dev)), X.to(dev))
    torch.cuda.synchronize()
    want = orc.gemv_q4_0_f32(qs.numpy(), np16(d), X.numpy())
    assert np.array_equal(npc(y).astype(np.float64), want)


def test_w4a16_batch_invariance(mm, dev):
    # each row of a B-row call against the same row in other calls: bit for
    # bit within one kernel family (the fp32 kernels: every B for K > 4096 and
    # B = 1 otherwise, each (row, b) sum in one order; the matrix-core kernel:
    # B >= 2 at K <= 4096, column b depending on x row b only), within
    # rounding across the two
    for N, K in ((2000, 2048), (700, 8192), (1300, 4096), (129, 2560), (65, 96),
                 (40, 11008)):
        W, _, _ = _q4(mm, N, K, dev, "inv")
        Bmax = min(8, mm.Q4F32_MAX_XK // K)
        X = synth.activations(Bmax, K, 0, "w4a16inv", K, device=dev)
        yB = mm.gemv_q4_0_f32(W, X)
        assert torch.equal(yB, mm.gemv_q4_0_f32(W, X))
        mf = K <= 4096 and Bmax >= 2
        for b in range(Bmax):
            y1 = mm.gemv_q4_0_f32(W, X[b].clone())
            if not mf:
                assert torch.equal(yB[b], y1)
                continue
            y2 = mm.gemv_q4_0_f32(W, X[[b, (b + 1) % Bmax]].clone())
            assert torch.equal(yB[b], y2[0])
            assert rel_l2_rows(npc(yB[b]), npc(y1).astype(np.float64)) <= 2e-5


@pytest.mark.parametrize("N,K", [(4096, 4096), (20000, 4096), (1000, 96), (777, 2560),
                                 (33, 32), (16, 512), (1, 128), (17, 32)])
def test_w4a16_both_kernels_every_b(mm, orc, dev, path, N, K):
    # the matrix-core kernel forced from B = 1 and the fp32 kernels forced at
    # every B, both against the oracle (20000 rows: several tiles per
    # workgroup on any GPU of up to 1250 compute units)
    W, qs, d = _q4(mm, N, K, dev, "both")
    for B in range(1, 9):
        X = synth.activations(B, K, 0, "w4a16both", N, K, B, device=dev)
        ref = orc.gemv_q4_0_f32(qs, d, npc(X))
        for sw in (1, -1):
            path(Q4F32_MF=sw)
            y = mm.gemv_q4_0_f32(W, X)
            torch.cuda.synchronize()
            # and the bound of the arithmetic: x kept to 2^-17 (bf16 hi + lo) in
            # both kernels, exact products, fp32 sums (rel-L2 ~5e-6 measured); a
            # lost lo part alone would give ~2^-9
            assert rel_l2_rows(npc(y), ref) <= W4A16_ARITH_TOL, (B, sw)


@pytest.mark.parametrize("N,K,B", [(1000, 11008, 1), (257, 9728, 1), (300, 14336, 1),
                                   (33, 16352, 1), (70, 6144, 2), (129, 2560, 1),
                                   (65, 3840, 1), (1000, 11008, 2), (129, 9728, 3),
                                   (300, 11008, 3), (70, 14336, 2), (300, 8192, 3),
                                   (4500, 8192, 3), (200, 2080, 1), (300, 18432, 2)])
def test_w4a16_ragged_rows(mm, orc, dev, N, K, B):
    # 64 < K/32 <= 512 blocks: the whole-row kernel with a ragged last step
    # (B <= 3; past B * K = 16384 only while its workgroups fit the CUs in one
    # round, so 4500 rows at B = 3 take the general kernel on a GPU of up to
    # 281 CUs; rows of 576 blocks always do, as 8-wave workgroups at B = 2
    # and 4-wave ones at B = 1), against the oracle; every row equals the
    # 1-row call on it
    # (same lanes per row, so the same bits in both kernels), and at B = 1
    # above K = 4096 the row of a call with enough x rows for the general
    # kernel
    W, qs, d = _q4(mm, N, K, dev, "ragged")
    Bg = 16384 // K + 1                      # rows that no longer fit the whole-row kernel at B = 1
    X = synth.activations(max(B, Bg), K, 0, "w4a16ragged", N, K, device=dev)
    y = mm.gemv_q4_0_f32(W, X[:B].clone())
    torch.cuda.synchronize()
    assert rel_l2_rows(npc(y), orc.gemv_q4_0_f32(qs, d, npc(X[:B]))) <= W4A16_ARITH_TOL
    if B > 1 and K > 4096:
        for b in range(B):
            assert torch.equal(y[b], mm.gemv_q4_0_f32(W, X[b].clone())), b
    if B == 1 and K > 4096 and Bg * K <= mm.Q4F32_MAX_XK:
        yg = mm.gemv_q4_0_f32(W, X[:Bg].clone())
        torch.cuda.synchronize()
        assert torch.equal(y, yg[:B])


@pytest.mark.parametrize("N,K,B", [(1, 4096, 1), (17, 11008, 1), (5, 28672, 1), (9, 11008, 2),
                                   (3, 8192, 3)])
def test_w4a16_fewer_rows_than_a_workgroup(mm, orc, dev, N, K, B):
    # the 8-wave workgroups (16 rows each) with fewer rows than that
    W, qs, d = _q4(mm, N, K, dev, "few")
    X = synth.activations(B, K, 0, "w4a16few", N, K, B, device=dev)
    y = mm.gemv_q4_0_f32(W, X)
    torch.cuda.synchronize()
    assert y.shape == (B, N)
    assert rel_l2_rows(npc(y), orc.gemv_q4_0_f32(qs, d, npc(X))) <= W4A16_ARITH_TOL


def test_w4a16_strided_x_and_y(mm, orc, dev):
    N, K, B = 1200, 1024, 5
    W, qs, d = _q4(mm, N, K, dev, "stride")
    Xb = synth.activations(B, K + 64, 0, "w4a16s", device=dev)
    X = Xb[:, 32:32 + K]
    Yb = torch.full((B, N + 7), 123.0, device=dev)
    mm.gemv_q4_0_f32(W, X, out=Yb[:, :N])
    torch.cuda.synchronize()
    ref = orc.gemv_q4_0_f32(qs, d, npc(X))
    assert rel_l2_rows(npc(Yb[:, :N]), ref) <= Q4_TOL
    assert torch.all(Yb[:, N:] == 123.0)
