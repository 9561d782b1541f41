"""Every entry point with its device buffers at legal offsets: 16-byte aligned
but not at the start of an allocation (48, 80 or 16 bytes in), on every
decode path, the routed products, the gated units, the router, dequant and the
prefill product.  Outputs start as NaN, so every element must be written; the
bars are the ones of the other parity tests (1e-3 * sum |w x| per element,
bit-exact dequant and routing)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from block_quantized_weight_q4_amd import synth

pytestmark = pytest.mark.gpu

TYPES = ("q4_0", "q4_k", "q6_k", "q5_k")
QK = {"q4_0": 32, "q4_k": 256, "q6_k": 256, "q5_k": 256}
BB = {"q4_0": 18, "q4_k": 144, "q6_k": 210, "q5_k": 176}


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


def at_offset(a: np.ndarray, off: int) -> torch.Tensor:
    """A device copy of `a` that starts `off` bytes into its allocation."""
    raw = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    buf = torch.zeros(raw.size + off + 64, dtype=torch.uint8, device="cuda")
    buf[off:off + raw.size] = torch.from_numpy(raw).cuda()
    return buf[off:off + raw.size]


def typed(t: torch.Tensor, dtype, shape) -> torch.Tensor:
    return t.view(dtype).view(*shape)


def nan_out(shape, dtype, off: int) -> torch.Tensor:
    n = int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size()
    buf = torch.zeros(n + off + 64, dtype=torch.uint8, device="cuda")
    out = buf[off:off + n].view(dtype).view(*shape)
    out.fill_(float("nan"))
    return out


def check_bound(y, yref, sa, what):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), what
    bad = np.abs(y - yref) > 1e-3 * sa
    assert not bad.any(), "%s: %d outside the bound" % (what, bad.sum())


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("B", [1, 2, 4, 9])
def test_matvec_offsets(gq, orc, t, B):
    """Both decode paths (batch 1, 2 on the dot path; 9 on the matrix cores;
    4 on either depending on the shape)."""
    g = synth.rng(0x6751000A, 10 * TYPES.index(t) + B)
    N, K = 301, 2 * QK[t] * 5
    W = synth.weight(t, g, N, K)
    x = synth.normal_f32(g, (B, K))
    bits = synth.bf16_bits(x)
    xb = synth.bf16_to_f32(bits)
    for xdt, xs, xt in (("f32", x, typed(at_offset(x, 48), torch.float32, (B, K))),
                        ("bf16", xb, typed(at_offset(bits, 80), torch.bfloat16, (B, K)))):
        y = nan_out((B, N), torch.float32, 16)
        gq.gq_matvec(t, at_offset(W, 48), N, K, xt, y)
        torch.cuda.synchronize()
        yref, sa = orc.matvec(t, W, N, K, xs)
        check_bound(y.cpu().numpy(), yref, sa, "%s B=%d %s" % (t, B, xdt))


@pytest.mark.parametrize("t", TYPES)
def test_dequant_offsets(gq, orc, t):
    g = synth.rng(0x6751000A, 100 + TYPES.index(t))
    blocks = synth.weight(t, g, 7, 3 * QK[t])
    out = nan_out((7 * 3 * QK[t],), torch.float32, 80)
    gq.gq_dequant(t, at_offset(blocks, 16), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), orc.dequant(t, blocks).view(np.uint32))


def test_routed_glu_router_offsets(gq, orc):
    """Router, gated unit and weighted down projection of a small MoE layer,
    every buffer off its allocation's start."""
    g = synth.rng(0x6751000A, 200)
    E, H, F, T, k = 12, 512, 256, 5, 3
    logits = synth.router_logits(g, T, E)
    ids = typed(at_offset(np.zeros((T, k), np.int32), 16), torch.int32, (T, k))
    rw = typed(at_offset(np.zeros((T, k), np.float32), 48), torch.float32, (T, k))
    gq.gq_route_topk(typed(at_offset(logits, 80), torch.float32, (T, E)), k, ids, rw)
    ids_ref, rw_ref = orc.route_topk(logits, k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    gate = synth.weight("q4_k", g, E * F, H)
    up = synth.weight("q4_k", g, E * F, H)
    down = synth.weight("q4_k", g, E * H, F)
    x = synth.normal_f32(g, (T, H))
    ws_n = gq.gq_matvec_id_workspace(E, T, k, H)
    ws = at_offset(np.zeros(ws_n, np.uint8), 16)
    h = nan_out((T, k, F), torch.float32, 48)
    gq.gq_matvec_id_glu("q4_k", at_offset(gate, 16), at_offset(up, 80), E, F, H, ids,
                        typed(at_offset(x, 48), torch.float32, (T, H)), "silu", h, ws)
    torch.cuda.synchronize()
    gg, sg = orc.matvec_id("q4_k", gate, E, F, H, ids_ref, x, False)
    uu, su = orc.matvec_id("q4_k", up, E, F, H, ids_ref, x, False)
    ref = orc.glu(gg, uu, "silu")
    ag = orc.glu(gg, np.ones_like(gg), "silu")
    bound = 1.2e-3 * sg * np.abs(uu) + 1e-3 * su * np.abs(ag) + 1.2e-6 * sg * su + 4e-6 * np.abs(ref)
    hv = h.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(hv)) and np.all(np.abs(hv - ref) <= bound)
    # the down projection, per slot and weighted, on the oracle's h (both
    # sides take the same input; the device's weights are its own routing's)
    h32 = ref.astype(np.float32)
    hin = typed(at_offset(h32, 80), torch.float32, (T, k, F))
    y = nan_out((T, H), torch.float32, 80)
    gq.gq_matvec_id("q4_k", at_offset(down, 48), E, H, F, ids, hin, True, y, ws, rw)
    y1 = nan_out((T, k, H), torch.float32, 16)
    gq.gq_matvec_id("q4_k", at_offset(down, 48), E, H, F, ids, hin, True, y1, ws)
    torch.cuda.synchronize()
    yref, sa = orc.matvec_id("q4_k", down, E, H, F, ids_ref, h32, True, rw_ref.astype(np.float32))
    check_bound(y.cpu().numpy(), yref, sa, "weighted down")
    yref1, sa1 = orc.matvec_id("q4_k", down, E, H, F, ids_ref, h32, True)
    check_bound(y1.cpu().numpy(), yref1, sa1, "per-slot down")
    assert gq.gq_matvec_id_check(ws) == 0


def test_dense_glu_offsets(gq, orc):
    g = synth.rng(0x6751000A, 300)
    N, K, B = 130, 1024, 3
    Wg = synth.weight("q6_k", g, N, K)
    Wu = synth.weight("q6_k", g, N, K)
    x = synth.normal_f32(g, (B, K))
    h = nan_out((B, N), torch.float32, 48)
    gq.gq_matvec_glu("q6_k", at_offset(Wg, 80), at_offset(Wu, 16), N, K,
                     typed(at_offset(x, 16), torch.float32, (B, K)), "gelu_tanh", h)
    torch.cuda.synchronize()
    gg, sg = orc.matvec("q6_k", Wg, N, K, x)
    uu, su = orc.matvec("q6_k", Wu, N, K, x)
    ref = orc.glu(gg, uu, "gelu_tanh")
    ag = orc.glu(gg, np.ones_like(gg), "gelu_tanh")
    bound = 1.2e-3 * sg * np.abs(uu) + 1e-3 * su * np.abs(ag) + 1.2e-6 * sg * su + 4e-6 * np.abs(ref)
    hv = h.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(hv)) and np.all(np.abs(hv - ref) <= bound)


@pytest.mark.parametrize("t", TYPES)
def test_matmul_offsets(gq, orc, t):
    """Prefill with W, X and Y off their allocations' starts (K >= 1024, where
    the prefill bar holds)."""
    g = synth.rng(0x6751000A, 400 + TYPES.index(t))
    M, N, K = 45, 72, 1024  # Y rows of 72 fp32 keep the 16-byte row alignment
    W = synth.weight(t, g, N, K)
    x = synth.normal_f32(g, (M, K))
    bits = synth.bf16_bits(x)
    X = typed(at_offset(bits, 48), torch.bfloat16, (M, K))
    Y = nan_out((M, N), torch.float32, 80)
    gq.gq_matmul(t, at_offset(W, 16), N, K, X, Y)
    torch.cuda.synchronize()
    yref, sa = orc.matmul_rows(t, W, N, K, synth.bf16_to_f32(bits), np.arange(M))
    check_bound(Y.cpu().numpy(), yref, sa, t)
