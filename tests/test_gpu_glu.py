"""GPU parity of gq_matvec_glu (gate and up products with the activation and
product between them, one launch) against the CPU oracle.

Bar: with g, u the oracle's exact products and S_g, S_u their sums
sum_k |w x| (the matvec bar is 1e-3 S per product),
  |h - act(g) u| <= 1.2e-3 S_g |u| + 1e-3 S_u |act(g)| + 1.2e-6 S_g S_u + 4e-6 |h|
(1.2 bounds |act'| for both activations; the last term covers fp32 exp/tanh
and the product), plus 2^-8 |h| for bf16 outputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from block_quantized_weight_q4_amd import synth

pytestmark = pytest.mark.gpu

TYPES = ("q4_0", "q4_k", "q6_k", "q5_k")
SHAPES = {"q4_0": [(37, 2816), (300, 704), (704, 2048)], "q4_k": [(130, 2560), (9, 4096), (705, 5120)],
          "q6_k": [(41, 1024), (333, 5120)], "q5_k": [(130, 2560), (64, 1024)]}


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


def make_x(g, B, K, xdt):
    x = synth.normal_f32(g, (B, K))
    if xdt == "bf16":
        bits = synth.bf16_bits(x)
        return synth.bf16_to_f32(bits), dev(bits.view(np.int16)).view(torch.bfloat16)
    return x, dev(x)


def run_glu(gq, t, Wg, Wu, N, K, x_t, B, act, hdt):
    h = torch.full((B, N), float("nan"), device="cuda", dtype=torch.float32 if hdt == "f32" else torch.bfloat16)
    gq.gq_matvec_glu(t, dev(Wg), dev(Wu), N, K, x_t, act, h)
    torch.cuda.synchronize()
    return h.float().cpu().numpy()


def check_glu(orc, t, Wg, Wu, N, K, x, h, act, hdt, what):
    g, sg = orc.matvec(t, Wg, N, K, x)
    u, su = orc.matvec(t, Wu, N, K, x)
    ref = orc.glu(g, u, act)
    ag = orc.glu(g, np.ones_like(g), act)
    bound = 1.2e-3 * sg * np.abs(u) + 1e-3 * su * np.abs(ag) + 1.2e-6 * sg * su + 4e-6 * np.abs(ref)
    if hdt == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(ref)
    assert np.all(np.isfinite(h)), what
    err = np.abs(h.astype(np.float64) - ref)
    bad = err > bound
    assert not bad.any(), "%s: %d outside the bound, first %s: h=%r ref=%r bound=%r" % (
        what, bad.sum(), np.argwhere(bad)[0], h[tuple(np.argwhere(bad)[0])], ref[tuple(np.argwhere(bad)[0])],
        bound[tuple(np.argwhere(bad)[0])])
    pos = bound > 0
    return float(np.max(err[pos] / bound[pos])) if pos.any() else 0.0


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
@pytest.mark.parametrize("xdt,hdt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_glu_parity(gq, orc, t, act, xdt, hdt):
    worst = 0.0
    for si, (N, K) in enumerate(SHAPES[t]):
        for B in (1, 3, 8):
            g = synth.rng(0x67510008, 1000 * TYPES.index(t) + 10 * B + si)
            Wg = synth.weight(t, g, N, K)
            Wu = synth.weight(t, g, N, K)
            x, x_t = make_x(g, B, K, xdt)
            h = run_glu(gq, t, Wg, Wu, N, K, x_t, B, act, hdt)
            worst = max(worst, check_glu(orc, t, Wg, Wu, N, K, x, h, act, hdt,
                                         "%s %s N=%d K=%d B=%d %s->%s" % (t, act, N, K, B, xdt, hdt)))
    print("worst error / bound = %.4f" % worst)


def test_glu_concatenated_gate_up_matrix(gq, orc):
    """W_gate and W_up as the two halves of one [2N] gate|up matrix."""
    t, N, K = "q4_k", 200, 2560
    g = synth.rng(0x67510008, 5000)
    W = synth.weight(t, g, 2 * N, K)
    Wd = dev(W)
    x, x_t = make_x(g, 2, K, "f32")
    h = torch.empty(2, N, device="cuda")
    gq.gq_matvec_glu(t, Wd[:N], Wd[N:], N, K, x_t, "silu", h)
    torch.cuda.synchronize()
    check_glu(orc, t, W[:N], W[N:], N, K, x, h.cpu().numpy(), "silu", "f32", "concatenated")


def test_glu_edge_cases(gq):
    h = torch.full((3, 7), float("nan"), device="cuda")
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    gq.gq_matvec_glu("q4_k", e, e, 7, 0, torch.empty(3, 0, device="cuda"), "gelu_tanh", h)
    torch.cuda.synchronize()
    assert torch.all(h == 0)
    h2 = torch.full((1, 4), 2.0, device="cuda")
    w = torch.empty(144, dtype=torch.uint8, device="cuda")
    gq.gq_matvec_glu("q4_k", w, w, 0, 256, torch.zeros(1, 256, device="cuda"), "silu", h2[:, :0])
    torch.cuda.synchronize()
    assert torch.all(h2 == 2.0)


@pytest.mark.parametrize("B", [1, 4])
def test_glu_workload_dense_ffn_hidden2560(gq, orc, B):
    """The hidden-2560 dense layer's FFN: gate and up 9728 x 2560 (Q4_K), fp32."""
    N, K = 9728, 2560
    Wg = synth.weight("q4_k", synth.rng(0x67510002, 4), N, K)
    Wu = synth.weight("q4_k", synth.rng(0x67510002, 5), N, K)
    x = synth.normal_f32(synth.rng(0x67510002, 400 + B), (B, K))
    h = run_glu(gq, "q4_k", Wg, Wu, N, K, dev(x), B, "silu", "f32")
    r = check_glu(orc, "q4_k", Wg, Wu, N, K, x, h, "silu", "f32", "dense FFN B=%d" % B)
    print("worst err/bound %.4f" % r)


@pytest.mark.parametrize("B", [1, 8])
def test_glu_workload_mixed_ffn_hidden5120_bf16(gq, orc, B):
    """The hidden-5120 layer's FFN: gate and up 17408 x 5120 (Q4_K), bf16 in and
    out (h feeds the Q6_K down projection as bf16)."""
    N, K = 17408, 5120
    Wg = synth.weight("q4_k", synth.rng(0x67510003, 4), N, K)
    Wu = synth.weight("q4_k", synth.rng(0x67510003, 5), N, K)
    x, x_t = make_x(synth.rng(0x67510003, 500 + B), B, K, "bf16")
    h = run_glu(gq, "q4_k", Wg, Wu, N, K, x_t, B, "gelu_tanh", "bf16")
    r = check_glu(orc, "q4_k", Wg, Wu, N, K, x, h, "gelu_tanh", "bf16", "mixed FFN B=%d" % B)
    print("worst err/bound %.4f" % r)
