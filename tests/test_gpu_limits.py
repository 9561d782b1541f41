"""GPU parity at the largest sizes the C ABI accepts: the longest row (K =
4,194,304 inputs: every decode path then tiles its activations many times
over and addresses rows of 2-3.4 MB through one buffer resource) and a
dequantisation whose output passes 2^32 bytes (64-bit element indexing).
Bars as in the other parity tests."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from block_quantized_weight_q4_amd import synth

pytestmark = pytest.mark.gpu

KMAX = 1 << 22


@pytest.fixture(autouse=True)
def _name_the_case(request):
    print("\n[gpu case] %s" % request.node.nodeid, flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def gq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_quantized_weight_q4_amd as g
    return g


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_bound(y, yref, sumabs, what):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), what
    bad = np.abs(y - yref) > 1e-3 * sumabs
    assert not bad.any(), "%s: %d elements outside the bound" % (what, bad.sum())


@pytest.mark.parametrize("t,B", [("q4_0", 1), ("q4_k", 1), ("q4_k", 5), ("q6_k", 2), ("q5_k", 1), ("q4_k", 9),
                                 ("q6_k", 9), ("q4_0", 6), ("q5_k", 8)])
def test_matvec_longest_row(gq, orc, t, B):
    """K = 2^22 with 37 rows (two and a bit workgroups of rows on every path):
    batch 1/2 on the dot-product path, 5..9 on the matrix cores."""
    N = 37
    g = synth.rng(0x67510009, ("q4_0", "q4_k", "q6_k", "q5_k").index(t) * 10 + B)
    W = synth.weight(t, g, N, KMAX)
    x = synth.normal_f32(g, (B, KMAX))
    y = torch.full((B, N), float("nan"), device="cuda")
    gq.gq_matvec(t, dev(W), N, KMAX, dev(x), y)
    torch.cuda.synchronize()
    yref, sa = orc.matvec(t, W, N, KMAX, x)
    check_bound(y.cpu().numpy(), yref, sa, "%s K=2^22 B=%d" % (t, B))


def test_matvec_id_longest_row(gq, orc):
    E, N, T, k = 3, 20, 2, 2
    g = synth.rng(0x67510009, 100)
    ex = synth.weight("q4_k", g, E * N, KMAX)
    ids = np.array([[2, 0], [2, 1]], np.int32)
    x = synth.normal_f32(g, (T, KMAX))
    ws = torch.empty(gq.gq_matvec_id_workspace(E, T, k, N), dtype=torch.uint8, device="cuda")
    y = torch.full((T, k, N), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_k", dev(ex), E, N, KMAX, dev(ids), dev(x), False, y, ws)
    torch.cuda.synchronize()
    yref, sa = orc.matvec_id("q4_k", ex, E, N, KMAX, ids, x, False)
    check_bound(y.cpu().numpy(), yref, sa, "matvec_id K=2^22")


def test_matmul_longest_row(gq, orc):
    """Prefill with the longest row it takes: the X row stride must stay below
    2^22 elements, so K = 2^22 - 256 with packed X rows; 5 rows of X, 70
    weight rows."""
    M, N, K = 5, 70, KMAX - 256
    g = synth.rng(0x67510009, 200)
    W = synth.weight("q4_k", g, N, K)
    x = synth.normal_f32(g, (M, K))
    bits = synth.bf16_bits(x)
    xf = synth.bf16_to_f32(bits)
    Y = torch.full((M, 72), float("nan"), device="cuda")  # row stride 72: 16-byte aligned rows
    gq.gq_matmul("q4_k", dev(W), N, K, dev(bits.view(np.int16)).view(torch.bfloat16), Y)
    torch.cuda.synchronize()
    yref, sa = orc.matmul_rows("q4_k", W, N, K, xf, np.arange(M))
    y = Y.cpu().numpy()
    check_bound(y[:, :N], yref, sa, "matmul K=2^22-256")
    assert np.all(np.isnan(y[:, N:]))


def test_dequant_output_past_4_gib(gq, orc):
    """2^22 + 3 Q4_K blocks -> 1,073,742,592 fp32 weights (4 GiB + 3 KiB): the
    last blocks, blocks around the 2^31 and 2^32 byte marks and a random
    sample are compared bit for bit with the oracle."""
    nb = (1 << 22) + 3
    g = synth.rng(0x67510009, 300)
    blocks = synth.blocks("q4_k", g, nb)
    out = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
    gq.gq_dequant("q4_k", dev(blocks), out)
    torch.cuda.synchronize()
    s = np.random.default_rng(5)
    pick = np.unique(np.concatenate([np.arange(nb - 8, nb), (1 << 21) + np.arange(-2, 3), (1 << 22) + np.arange(-2, 3),
                                     s.integers(0, nb, 64)]))
    for b in pick:
        ref = orc.dequant("q4_k", blocks[b])
        got = out[int(b) * 256:(int(b) + 1) * 256].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), int(b)
