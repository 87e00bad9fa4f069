"""Test helpers: comparisons, tensor conversions and MoE layer builders that
hand the same synthetic bytes to the HIP library and to the oracle."""
from __future__ import annotations

import numpy as np
import torch

import synth


def rel_l2_rows(y, ref):
    """max over rows of ||y_b - ref_b||_2 / ||ref_b||_2 (float64)."""
    y = np.atleast_2d(np.asarray(y, np.float64))
    ref = np.atleast_2d(np.asarray(ref, np.float64))
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def np16(t: torch.Tensor) -> np.ndarray:
    """16-bit tensor (bf16 / f16 / int16) -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def npc(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


def f16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(device)


def logit_bound(R: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Forward error bound of an fp32 router logit: each lane sums H/64 products
    in sequence, then a 64-lane tree; gamma = (H/64 + 8) * 2^-24, doubled."""
    H = R.shape[1]
    gamma = 2 * (H / 64 + 8) * 2.0 ** -24
    return gamma * (np.abs(X.astype(np.float64)) @ np.abs(R.astype(np.float64)).T)


def build_moe(mm, orc, E, H, I, k, seed, *tags, shared=True, shared_gate=False, device="cuda"):
    """(library MoeLayer on device, oracle MoE on host) from one set of synthetic tensors."""
    t = synth.moe_layer_tensors(E, H, I, seed, *tags, shared=shared, shared_gate=shared_gate,
                                device=device)
    sh = t.get("shared")
    layer = mm.MoeLayer(t["router"], t["gate_qs"], t["gate_d"], t["up_qs"], t["up_d"],
                        t["down_qs"], t["down_d"], k, shared=sh,
                        shared_gate_row=t.get("shared_gate_row"))
    sh_np = None
    if sh is not None:
        sh_np = (npc(sh["gate_qs"]), np16(sh["gate_d"]), npc(sh["up_qs"]), np16(sh["up_d"]),
                 npc(sh["down_qs"]), np16(sh["down_d"]))
    sgr = t.get("shared_gate_row")
    ref = orc.MoE(npc(t["router"]), npc(t["gate_qs"]), np16(t["gate_d"]), npc(t["up_qs"]),
                  np16(t["up_d"]), npc(t["down_qs"]), np16(t["down_d"]), k, shared=sh_np,
                  shared_gate_row=None if sgr is None else npc(sgr))
    return layer, ref


def check_route(orc, R, X, logits_gpu, ids_gpu, k, E):
    """Router parity: logits within the forward-error bound of the float64
    oracle; ids bit-exact against the oracle's top-k taken on the GPU's own fp32
    logits (same-precision decision); ids equal to the oracle's float64-based
    ids except where the float64 logits are within twice the bound of each
    other at a differing rank.  Returns the number of such near-tie rows."""
    ref = orc.router_logits(R, X)
    bound = logit_bound(R, X)
    lg = logits_gpu[:, :E].astype(np.float64)
    assert (np.abs(lg - ref) <= bound).all(), float(np.abs(lg - ref).max())
    assert np.array_equal(ids_gpu, orc.topk(logits_gpu[:, :E].astype(np.float32), k))
    ids_ref = orc.topk(ref.astype(np.float32), k)
    near = 0
    for b in range(X.shape[0]):
        if np.array_equal(ids_ref[b], ids_gpu[b]):
            continue
        # every differing rank must be a near tie in float64
        order = np.lexsort((np.arange(E), -ref[b]))
        vals = ref[b][order]
        diff = [j for j in range(k) if ids_ref[b, j] != ids_gpu[b, j]]
        for j in diff:
            lo = max(j - 1, 0)
            gap = np.abs(np.diff(vals[lo:min(j + 2, E)])).min()
            assert gap <= 2 * bound[b].max(), (b, j, gap)
        near += 1
    return near


def check_ids_admissible(orc, R, X, ids_gpu, k):
    """Every row's ids must be a top-k that fp32 rounding of the logits could
    produce: distinct and in [0, E); each selected logit (float64) at least
    every unselected one minus twice the forward-error bound; consecutive
    slots in descending order up to the same margin.  Rows equal to the
    float64 top-k pass trivially.  Returns (float64 logits, rows whose ids
    differ from the float64 top-k)."""
    ref = orc.router_logits(R, X)
    bound = logit_bound(R, X)
    E = R.shape[0]
    ids_ref = orc.topk(ref.astype(np.float32), k)
    differ = []
    for b in range(X.shape[0]):
        sel = ids_gpu[b].astype(np.int64)
        assert ((sel >= 0) & (sel < E)).all(), (b, sel)
        assert len(set(sel.tolist())) == k, (b, sel)
        if np.array_equal(sel, ids_ref[b]):
            continue
        differ.append(b)
        margin = 2 * bound[b].max()
        lv = ref[b][sel]
        rest = np.delete(ref[b], sel)
        assert rest.size == 0 or lv.min() >= rest.max() - margin, (b, lv.min(), rest.max())
        assert (np.diff(lv) <= margin).all(), (b, lv)
    return ref, differ


def moe_ref_with_ids(orc, ref, X, ids, logits64):
    """The oracle's layer output for the given routing (ids taken as given):
    weights from the float64 logits renormalised over those ids, gate/up,
    Q8_1(h), down and the combine."""
    w64 = orc.gate_weights(logits64, ids)
    B = X.shape[0]
    if ref.shared_gate_row is not None:
        z = X.astype(np.float64) @ ref.shared_gate_row.astype(np.float64)
        s64 = 1.0 / (1.0 + np.exp(-z))
    else:
        s64 = np.ones(B)
    h = ref.gate_up(X, ids)
    hq, hds = orc.quantize_q8_1(h)
    return ref.down(hq, hds, ids, w64, s64)


# ---------------------------------------------------------------------------
# interchange blocks (array-of-structures) <-> the library's planar layout
# ---------------------------------------------------------------------------

def q8_1_to_blocks(codes: np.ndarray, ds: np.ndarray) -> np.ndarray:
    """Planar Q8_1 (codes int8 [B, K], ds uint16 [B, K/32, 2]) -> 36-byte
    blocks uint8 [B, K/32, 36]: d, s (fp16, little endian), 32 codes."""
    B, K = codes.shape
    nb = K // 32
    out = np.empty((B, nb, 36), np.uint8)
    out[:, :, :4] = np.ascontiguousarray(ds.reshape(B, nb, 2)).astype("<u2").view(np.uint8)
    out[:, :, 4:] = np.ascontiguousarray(codes.reshape(B, nb, 32)).view(np.uint8)
    return out


def q8_1_from_blocks(blocks: np.ndarray):
    """36-byte Q8_1 blocks uint8 [B, nb, 36] -> planar (codes int8 [B, 32 nb],
    ds uint16 [B, nb, 2])."""
    B, nb, _ = blocks.shape
    ds = np.ascontiguousarray(blocks[:, :, :4]).view("<u2").reshape(B, nb, 2).astype(np.uint16)
    codes = np.ascontiguousarray(blocks[:, :, 4:]).view(np.int8).reshape(B, nb * 32)
    return codes, ds


def q4_0_to_blocks(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Planar Q4_0 (qs uint8 [N, K/32, 16], d uint16 [N, K/32]) -> 18-byte
    blocks uint8 [N, K/32, 18]: d (fp16, little endian), 16 code bytes."""
    N, nb, _ = qs.shape
    out = np.empty((N, nb, 18), np.uint8)
    out[:, :, :2] = np.ascontiguousarray(d).astype("<u2").view(np.uint8).reshape(N, nb, 2)
    out[:, :, 2:] = qs
    return out


def q4_0_from_blocks(blocks: np.ndarray):
    """18-byte Q4_0 blocks uint8 [N, nb, 18] -> planar (qs uint8 [N, nb, 16],
    d uint16 [N, nb])."""
    N, nb, _ = blocks.shape
    d = np.ascontiguousarray(blocks[:, :, :2]).view("<u2").reshape(N, nb).astype(np.uint16)
    return np.ascontiguousarray(blocks[:, :, 2:]), d


def read_golden_blocks(path):
    """{name: uint8 array} of the hex lines of a golden block file."""
    out = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            name, *hexes = line.split()
            out[name] = np.array([int(h, 16) for h in hexes], np.uint8)
    return out


def q8_1_halfway_blocks(orc, n, seed=0):
    """n blocks of 32 fp32 values (rows of an array [n, 32]) whose Q8_1 block
    sum is a rounding boundary: the fp32 product d32 * sum(q) lies exactly
    halfway between two fp16 values while the exact product does not, so
    rounding the fp32 product to fp16 (the definition) and rounding the exact
    product once give different bits.  Found by a seeded search with the
    oracle's codes."""
    rng = np.random.default_rng(seed)
    found = []
    while len(found) < n:
        x = rng.standard_normal((1 << 16, 32)).astype(np.float32)
        q, _ = orc.quantize_q8_1(x.reshape(1, -1))
        S = q.reshape(-1, 32).astype(np.int64).sum(1)
        d32 = (np.abs(x).max(1) / np.float32(127.0)).astype(np.float32)
        p32 = (d32 * S.astype(np.float32)).astype(np.float32)
        exact = d32.astype(np.float64) * S
        differ = p32.astype(np.float16).view(np.uint16) != exact.astype(np.float16).view(np.uint16)
        found.extend(x[differ][: n - len(found)])
    return np.stack(found[:n])
