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
