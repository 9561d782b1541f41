"""GPU parity of gq_route_topk (softmax + top-k routing) against the CPU oracle.

Bars: ids bit-exact (the choice compares fp32 logits on both sides); weights
within (top_k + 8) * 2^-24 of the oracle's fp64 softmax: each exp carries a few
fp32 roundings relative to its value (<= 1), the sum about top_k of them and
the division one more."""
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


def route(gq, logits_np, k):
    T = logits_np.shape[0]
    lg = torch.from_numpy(np.ascontiguousarray(logits_np, np.float32)).cuda()
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), device="cuda")
    gq.gq_route_topk(lg, k, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check(gq, orc, logits, k, what):
    ids, w = route(gq, logits, k)
    rid, rw = orc.route_topk(logits, k)
    bad = np.argwhere(ids != rid)
    assert bad.size == 0, "%s: ids differ first at %s: %s vs %s" % (what, bad[0], ids[bad[0][0]], rid[bad[0][0]])
    err = np.abs(w.astype(np.float64) - rw)
    assert np.all(np.isfinite(w)), what
    assert err.max() <= (k + 8) * 2.0 ** -24, "%s: weight error %g" % (what, err.max())
    return err.max()


def test_moe_router_8_tokens_128_experts_top8(gq, orc):
    g = synth.rng(0x67510004, 0)
    logits = synth.router_logits(g, 8, 128)
    e = check(gq, orc, logits, 8, "moe")
    print("max weight error %.3g" % e)


@pytest.mark.parametrize("E,k", [(1, 1), (5, 3), (64, 64), (65, 7), (128, 8), (129, 64), (300, 17),
                                 (1000, 64), (4096, 1), (4096, 64)])
def test_route_shapes(gq, orc, E, k):
    g = synth.rng(0x67510005, E * 100 + k)
    for T in (1, 3, 4, 5, 37):
        logits = (2.0 * g.standard_normal((T, E))).astype(np.float32)
        check(gq, orc, logits, k, "E=%d k=%d T=%d" % (E, k, T))


def test_route_ties_signed_zeros_and_extremes(gq, orc):
    """Many equal logits (rounded values), -0 next to +0, infinities and
    magnitudes near the fp32 limit: ids must follow the lower-id tie rule."""
    g = synth.rng(0x67510005, 1)
    T, E = 64, 256
    logits = np.round(g.standard_normal((T, E)), 0).astype(np.float32)
    logits[0, :] = 0.0
    logits[0, 1::2] = -0.0
    logits[1, :] = -np.inf
    logits[1, 77] = 3.0e38
    logits[1, 200] = -3.0e38
    logits[2, 5:9] = 3.0e38
    logits[3, ::3] = -np.inf
    logits[4, :] = 1e-45  # subnormal ties
    logits[4, 130] = 2e-45
    for k in (1, 8, 64):
        check(gq, orc, logits, k, "ties k=%d" % k)


def test_route_prefill_sized_batch(gq, orc):
    """3015 tokens (the prefill length) routed 8 of 128: every token checked."""
    g = synth.rng(0x67510005, 2)
    logits = synth.router_logits(g, 3015, 128)
    check(gq, orc, logits, 8, "prefill")


def test_route_no_tokens_is_a_no_op(gq):
    lg = torch.empty((0, 128), device="cuda")
    ids = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 8), device="cuda")
    gq.gq_route_topk(lg, 8, ids, w)
    torch.cuda.synchronize()
