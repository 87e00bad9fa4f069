"""The allocation-free MoE entry point (moe_layer_decode_noalloc) against the
workspace one (moe_layer_decode): the same kernels, so the same bits, on two
calls in a row, the second with fewer rows; and the oracle's layer."""
import numpy as np
import pytest
import torch

import synth
from tests._util import build_moe, check_ids_admissible, moe_ref_with_ids, npc, rel_l2_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("E,H,I,k,Bs", [(512, 2048, 512, 10, (8, 2)),
                                        (256, 2048, 512, 8, (3, 1)),
                                        (64, 512, 64, 6, (40, 12))])
def test_noalloc_matches_workspace_entry(mm, orc, dev, E, H, I, k, Bs):
    layer, ref = build_moe(mm, orc, E, H, I, k, 0, "noalloc", E, H, I, device=dev)
    for B in Bs:     # two calls in a row, the second with fewer rows
        X = synth.activations(B, H, 0, "noalloc", E, B, device=dev)
        ids_a = torch.empty((B, k), dtype=torch.int32, device=dev)
        ids_b = torch.empty((B, k), dtype=torch.int32, device=dev)
        w_b = torch.empty((B, k), dtype=torch.float32, device=dev)
        y_ws = mm.moe_layer_decode(layer, X, ids=ids_a)
        y_na = mm.moe_layer_decode_noalloc(layer, X, ids=ids_b, weights=w_b)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), B
        assert torch.equal(ids_b, ids_a), B
        ids_np = npc(ids_b)
        lg64, differ = check_ids_admissible(orc, ref.router, npc(X), ids_np, k)
        assert len(differ) <= max(1, B // 8)
        assert rel_l2_rows(npc(y_na), moe_ref_with_ids(orc, ref, npc(X), ids_np, lg64)) <= 2e-3
    # without ids / weights outputs (the routing stays in the library's array)
    y2 = mm.moe_layer_decode_noalloc(layer, X)
    torch.cuda.synchronize()
    assert torch.equal(y2, y_na)
