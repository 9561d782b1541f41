"""GPU: gq_matvec_id_noalloc (the routed product on the library's own per-GPU
workspace) against gq_matvec_id with a caller workspace, bit for bit: an
unweighted and a weighted call, then -- on the same array, which keeps the
last call's contents -- a smaller call, a call that reuses the previous call's
group table, and an oversized request that must be refused."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from block_quantized_weight_q4_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    print("\n[gpu case] %s" % request.node.nodeid, flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def gq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_quantized_weight_q4_amd as g
    return g


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def both(gq, t, ex, E, N, K, ids, x, per_slot, rw):
    """(noalloc result, workspace result) of the same call."""
    T, k = ids.shape
    shape = (T, N) if rw is not None else (T, k, N)
    ya = torch.full(shape, float("nan"), device="cuda")
    gq.gq_matvec_id_noalloc(t, ex, E, N, K, ids, x, per_slot, ya, rw)
    ws = torch.empty(gq.gq_matvec_id_workspace(E, T, k, N), dtype=torch.uint8, device="cuda")
    yb = torch.full(shape, float("nan"), device="cuda")
    gq.gq_matvec_id(t, ex, E, N, K, ids, x, per_slot, yb, ws, rw)
    torch.cuda.synchronize()
    return ya, yb


def test_noalloc_matches_workspace_call(gq):
    g = synth.rng(0x67510004, 90)
    E, H, F = 128, 2816, 704
    gate = dev(synth.weight("q4_0", synth.rng(0x67510004, 1), E * F, H))
    down = dev(synth.weight("q4_0", synth.rng(0x67510004, 3), E * H, F))
    for T, k in ((8, 8), (3, 8)):  # the second call is smaller than the first
        logits = dev(synth.router_logits(g, T, E))
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        rw = torch.empty((T, k), device="cuda")
        gq.gq_route_topk(logits, k, ids, rw)
        x = dev(synth.normal_f32(g, (T, H)))
        ya, yb = both(gq, "q4_0", gate, E, F, H, ids, x, False, None)
        assert bool(torch.isfinite(ya).all())
        assert torch.equal(ya.view(torch.int32), yb.view(torch.int32)), (T, k, "gate")
        h = dev(synth.normal_f32(g, (T, k, F)))
        ya, yb = both(gq, "q4_0", down, E, H, F, ids, h, True, rw)
        assert bool(torch.isfinite(ya).all())
        assert torch.equal(ya.view(torch.int32), yb.view(torch.int32)), (T, k, "down")
        # the weighted call again, reusing the group table the last call left
        yr = torch.full((T, H), float("nan"), device="cuda")
        gq.gq_matvec_id_noalloc("q4_0", down, E, H, F, (T, k), h, True, yr, rw)
        torch.cuda.synchronize()
        assert torch.equal(yr.view(torch.int32), yb.view(torch.int32)), (T, k, "reused table")


def test_noalloc_refuses_oversized_workspace(gq):
    E, N, K, T, k = 16, 8192, 256, 128, 8  # 1024 slots x 8192 outputs: 32 MiB of per-slot rows
    ex = torch.zeros(E * N * (K // 256) * 144, dtype=torch.uint8, device="cuda")
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    x = torch.zeros((T, K), device="cuda")
    y = torch.full((T, N), 7.0, device="cuda")
    rw = torch.ones((T, k), device="cuda")
    with pytest.raises(gq.GqError, match="workspace"):
        gq.gq_matvec_id_noalloc("q4_k", ex, E, N, K, ids, x, False, y, rw)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
