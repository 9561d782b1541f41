"""GPU parity of every launch configuration bench.py times, against the oracle.

The launches come from block_quantized_weight_q4_amd.workloads, the same lists
bench.py builds its timed region from (block type, N, K, number of vectors,
activation type -- which decide the kernel variant and its launch shape), with
the same seeded inputs.  Outputs start as NaN, so every element must have been
written; the oracle computes all rows of the smaller launches and 16 sampled
runs of 64 rows (the first and last among them) of the larger ones, each
compared element by element within 1e-3 * sum_k |w x|."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_quantized_weight_q4_amd import synth, workloads
from tests.test_gpu_dequant_matvec import _name_the_case, check_bound, dev, gq  # noqa: F401
from tests.test_gpu_matvec_id_glu import check as glu_check, glu_ref

pytestmark = pytest.mark.gpu

FULL_MACS = 60_000_000  # above this many multiply-adds the oracle samples row runs


def sampled_rows(N: int, K: int, B: int, seed: int) -> list[tuple[int, int]]:
    if N * K * B <= FULL_MACS or N <= 1024:
        return [(0, N)]
    s = np.random.default_rng(seed)
    starts = sorted(set([0, N - 64] + [int(v) for v in s.choice(np.arange(64, N - 128), 14, replace=False)]))
    return [(a, min(a + 64, N)) for a in starts]


def x_tensor(x: np.ndarray, xdt: str) -> torch.Tensor:
    if xdt == "bf16":
        return dev(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16)
    return dev(x)


@pytest.mark.parametrize("L", workloads.TIMED_MATVEC, ids=lambda L: L.id)
def test_timed_matvec_launch(gq, orc, L):
    W = L.weight()
    assert W.shape[0] == L.N
    x = L.x()
    y = torch.full((L.batch, L.N), float("nan"), device="cuda")
    gq.gq_matvec(L.t, dev(W), L.N, L.K, x_tensor(x, L.xdt), y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "an output element was not written"
    y = y.cpu().numpy()
    worst = 0.0
    for r0, r1 in sampled_rows(L.N, L.K, L.batch, workloads.hash_name(L.id)):
        yref, sa = orc.matvec(L.t, W, L.N, L.K, x, rows=(r0, r1))
        worst = max(worst, check_bound(y[:, r0:r1], yref[:, r0:r1], sa[:, r0:r1], "%s rows %d..%d" % (L.id, r0, r1)))
    print("%s worst err/bound %.4f" % (L.id, worst))


@pytest.mark.parametrize("G", workloads.TIMED_GLU, ids=lambda G: G.id)
def test_timed_glu_launch(gq, orc, G):
    """h = act(gate x) * (up x), bar as in test_gpu_glu (derived from the matvec
    bar on both products through |act'| <= 1.2)."""
    Wg, Wu = G.weights()
    x = G.x()
    h = torch.full((G.batch, G.N), float("nan"), device="cuda")
    gq.gq_matvec_glu(G.t, dev(Wg), dev(Wu), G.N, G.K, dev(x), G.act, h)
    torch.cuda.synchronize()
    h = h.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(h))
    g, sg = orc.matvec(G.t, Wg, G.N, G.K, x)
    u, su = orc.matvec(G.t, Wu, G.N, G.K, x)
    ref = orc.glu(g, u, G.act)
    act_g = orc.glu(g, np.ones_like(u), G.act)
    bound = 1.2e-3 * sg * np.abs(u) + 1e-3 * su * np.abs(act_g) + 1.2e-6 * sg * su + 4e-6 * np.abs(ref)
    err = np.abs(h - ref)
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("m", [workloads.MOE, workloads.MoeLayer(T=64)], ids=["tokens8", "tokens64"])
def test_timed_moe_layer(gq, orc, m):
    """The routed-expert workload exactly as timed (8 tokens, and the fused
    layer's 64-token block): device routing of the seeded logits, gate and up
    per token (fp32 x), the weighted down projection of seeded per-slot h
    (fp32) and of the bf16 h the routed gated unit writes."""
    ex = m.experts()
    logits = m.logits()
    ids_t = torch.empty((m.T, m.k), dtype=torch.int32, device="cuda")
    rw_t = torch.empty((m.T, m.k), device="cuda")
    gq.gq_route_topk(dev(logits), m.k, ids_t, rw_t)
    torch.cuda.synchronize()
    ids, rw64 = orc.route_topk(logits, m.k)
    assert np.array_equal(ids_t.cpu().numpy(), ids)
    rw = rw_t.cpu().numpy()
    x = m.x()
    ws = torch.empty(max(gq.gq_matvec_id_workspace(m.E, m.T, m.k, m.F), gq.gq_matvec_id_workspace(m.E, m.T, m.k, m.H)),
                     dtype=torch.uint8, device="cuda")
    for name in ("gate", "up"):
        y = torch.full((m.T, m.k, m.F), float("nan"), device="cuda")
        gq.gq_matvec_id(m.t, dev(ex[name]), m.E, m.F, m.H, ids_t, dev(x), False, y, ws)
        torch.cuda.synchronize()
        yref, sa = orc.matvec_id(m.t, ex[name], m.E, m.F, m.H, ids, x, False)
        check_bound(y.cpu().numpy(), yref, sa, name)
    h = m.h()
    y = torch.full((m.T, m.H), float("nan"), device="cuda")
    gq.gq_matvec_id(m.t, dev(ex["down"]), m.E, m.H, m.F, ids_t, dev(h), True, y, ws, rw_t)
    torch.cuda.synchronize()
    yref, sa = orc.matvec_id(m.t, ex["down"], m.E, m.H, m.F, ids, h, True, rw)
    check_bound(y.cpu().numpy(), yref, sa, "down (seeded h)")
    # routing and the routed gated unit -> bf16 h -> weighted down, as in the
    # fused timed layer (the down product on the table the first call left)
    ids_t.fill_(-7)
    rw_t.fill_(float("nan"))
    hb = torch.full((m.T, m.k, m.F), float("nan"), device="cuda", dtype=torch.bfloat16)
    gq.gq_route_matvec_id_glu(m.t, dev(ex["gate"]), dev(ex["up"]), m.E, m.F, m.H, dev(logits), m.k, ids_t, rw_t,
                              dev(x), "silu", hb, ws)
    torch.cuda.synchronize()
    assert np.array_equal(ids_t.cpu().numpy(), ids)
    assert np.array_equal(rw_t.cpu().numpy().view(np.uint32), rw.view(np.uint32))
    hbits = hb.view(torch.int16).cpu().numpy().view(np.uint16)
    hf = synth.bf16_to_f32(hbits)
    # h against the oracle's gated unit, with the routed gated unit's bound
    href, hbound = glu_ref(orc, m.t, ex["gate"], ex["up"], m.E, m.F, m.H, ids, x, "silu", "bf16")
    glu_check(hf, href, hbound, "routed gated unit h (bf16)")
    # the down projection as timed: it reuses the group table the gated call
    # left in ws; the result equals a call that builds its own, bit for bit
    y = torch.full((m.T, m.H), float("nan"), device="cuda")
    gq.gq_matvec_id(m.t, dev(ex["down"]), m.E, m.H, m.F, (m.T, m.k), hb, True, y, ws, rw_t)
    y2 = torch.full((m.T, m.H), float("nan"), device="cuda")
    gq.gq_matvec_id(m.t, dev(ex["down"]), m.E, m.H, m.F, ids_t, hb, True, y2, ws, rw_t)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    yref, sa = orc.matvec_id(m.t, ex["down"], m.E, m.H, m.F, ids, hf, True, rw)
    check_bound(y.cpu().numpy(), yref, sa, "down (bf16 h of the routed gated unit)")


@pytest.mark.parametrize("L", workloads.TIMED_MATMUL, ids=lambda L: L.id)
def test_timed_prefill_launch(gq, orc, L):
    """Every timed prefill product at its full size: Y starts as NaN and must be
    finite everywhere afterwards (every element written); 64 sampled full rows
    (rows 0 and M-1, 8 of them in the last partial 256-row tile), 16 sampled
    full columns, a Freivalds checksum u^T Y v and the plain sum of Y against
    the oracle's closed forms."""
    M, N, K = L.M, L.N, L.K
    W = L.weight()
    xb = L.x_bf16_bits()
    xf = synth.bf16_to_f32(xb)
    X = dev(xb.view(np.int16)).view(torch.bfloat16)
    Y = torch.full((M, N), float("nan"), device="cuda")
    gq.gq_matmul(L.t, dev(W), N, K, X, Y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y).all()), "an output element was not written"
    s = np.random.default_rng(0x5EED + N)
    last = (M // 256) * 256
    rows = np.unique(np.concatenate([[0, M - 1], s.choice(np.arange(last, M - 1), 8, replace=False),
                                     s.choice(np.arange(1, last), 54, replace=False)]))
    assert rows.size == 64
    cols = np.unique(np.concatenate([[0, N - 1], s.choice(np.arange(1, N - 1), 14, replace=False)]))
    ref, sa = orc.matmul_rows(L.t, W, N, K, xf, rows)
    r1 = check_bound(Y[torch.from_numpy(rows).cuda()].cpu().numpy(), ref, sa, "sampled rows")
    refc, sac = orc.matmul_cols(L.t, W, N, K, xf, cols)
    r2 = check_bound(Y[:, torch.from_numpy(cols).cuda()].cpu().numpy(), refc, sac, "sampled columns")
    Yd = Y.double()
    u = s.choice([-1.0, 1.0], M)
    v = s.choice([-1.0, 1.0], N)
    got = float(torch.from_numpy(u).cuda() @ Yd @ torch.from_numpy(v).cuda())
    want, tol = orc.matmul_checksum(L.t, W, N, K, xf, u, v)
    assert abs(got - want) <= 1e-3 * tol, (got, want, tol)
    got1 = float(Yd.sum())
    want1, tol1 = orc.matmul_checksum(L.t, W, N, K, xf, np.ones(M), np.ones(N))
    assert abs(got1 - want1) <= 1e-3 * tol1, (got1, want1, tol1)
    print("%s rows worst %.4f cols worst %.4f" % (L.id, r1, r2))
