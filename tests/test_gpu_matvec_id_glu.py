"""GPU parity of gq_matvec_id_glu (routed gate and up products with the
activation and product between them, one launch) against the CPU oracle.

Bar, per slot (t, j) and row n, with g, u the oracle's exact routed products
and S_g, S_u their sums sum_k |w x| (the routed-product bar is 1e-3 S):
  |h - act(g) u| <= 1.2e-3 S_g |u| + 1e-3 S_u |act(g)| + 1.2e-6 S_g S_u + 4e-6 |h|
(1.2 bounds |act'| for both activations; the last term covers fp32 exp/tanh
and the product), plus 2^-8 |h| for bf16 outputs -- the bar of the dense
gated unit, applied to the routed products.

The MoE layer test then runs the whole routed feed-forward block on the
device (route, gated unit, weighted down projection) and checks the layer
output against the oracle's layer, with the gated unit's bound carried through
the down projection: sum_j |r_j| sum_k |w_down[n][k]| bound_h[t][j][k]."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from block_quantized_weight_q4_amd import synth

pytestmark = pytest.mark.gpu

TYPES = ("q4_0", "q4_k", "q6_k", "q5_k")
BB = {"q4_0": 18, "q4_k": 144, "q6_k": 210, "q5_k": 176}
QK = {"q4_0": 32, "q4_k": 256, "q6_k": 256, "q5_k": 256}


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


def make_x(g, shape, xdt):
    x = synth.normal_f32(g, shape)
    if xdt == "bf16":
        bits = synth.bf16_bits(x)
        return synth.bf16_to_f32(bits), dev(bits.view(np.int16)).view(torch.bfloat16)
    return x, dev(x)


def run_glu_id(gq, t, gate, up, E, N, K, ids, x_t, act, hdt):
    T, k = ids.shape
    ws = torch.empty(gq.gq_matvec_id_workspace(E, T, k, N), dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)  # contents need no initialisation
    h = torch.full((T, k, N), float("nan"), device="cuda", dtype=torch.float32 if hdt == "f32" else torch.bfloat16)
    gq.gq_matvec_id_glu(t, dev(gate), dev(up), E, N, K, dev(ids), x_t, act, h, ws)
    torch.cuda.synchronize()
    return h, ws


def glu_ref(orc, t, gate, up, E, N, K, ids, x, act, hdt):
    """(act(g) u, its per-element bound) from the oracle's routed products."""
    g, sg = orc.matvec_id(t, gate, E, N, K, ids, x, False)
    u, su = orc.matvec_id(t, up, E, N, K, ids, x, False)
    ref = orc.glu(g, u, act)
    ag = orc.glu(g, np.ones_like(g), act)
    bound = 1.2e-3 * sg * np.abs(u) + 1e-3 * su * np.abs(ag) + 1.2e-6 * sg * su + 4e-6 * np.abs(ref)
    if hdt == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(ref)
    return ref, bound


def check(h, ref, bound, what):
    h = np.asarray(h, np.float64)
    assert np.all(np.isfinite(h)), what
    err = np.abs(h - ref)
    bad = err > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d outside the bound, first %s: h=%r ref=%r bound=%r" % (
            what, bad.sum(), i, h[i], ref[i], bound[i]))
    pos = bound > 0
    return float(np.max(err[pos] / bound[pos])) if pos.any() else 0.0


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("xdt,hdt", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_glu_id_shapes(gq, orc, t, xdt, hdt):
    """Ragged row counts (several row tiles and a partial one), groups of one to
    several slots per expert, both activations."""
    worst = 0.0
    g = synth.rng(0x67510009, 10 * TYPES.index(t) + ["f32", "bf16"].index(xdt) + 2 * ["f32", "bf16"].index(hdt))
    cases = ((5, 37, 512, 3, 2), (16, 130, 1024, 6, 4), (9, 64, 2048, 16, 3), (4, 200, 256, 5, 4))
    for ci, (E, N, K, T, k) in enumerate(cases):
        gate = synth.weight(t, g, E * N, K)
        up = synth.weight(t, g, E * N, K)
        ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        x, x_t = make_x(g, (T, K), xdt)
        act = ("silu", "gelu_tanh")[ci % 2]
        h, ws = run_glu_id(gq, t, gate, up, E, N, K, ids, x_t, act, hdt)
        ref, bound = glu_ref(orc, t, gate, up, E, N, K, ids, x, act, hdt)
        worst = max(worst, check(h.float().cpu().numpy(), ref, bound,
                                 "%s E=%d N=%d K=%d T=%d k=%d %s %s->%s" % (t, E, N, K, T, k, act, xdt, hdt)))
        assert gq.gq_matvec_id_check(ws) == 0
    print("worst error / bound = %.4f" % worst)


def test_glu_id_repeated_experts_and_determinism(gq, orc):
    """Skewed routing (most slots to two experts, so long runs split into many
    groups); repeated calls are bit-identical."""
    g = synth.rng(0x67510009, 100)
    E, N, K, T, k = 32, 72, 768, 64, 4
    gate = synth.weight("q4_k", g, E * N, K)
    up = synth.weight("q4_k", g, E * N, K)
    ids = np.where(g.random((T, k)) < 0.7, g.integers(0, 2, (T, k)), g.integers(0, E, (T, k))).astype(np.int32)
    x, x_t = make_x(g, (T, K), "f32")
    h1, _ = run_glu_id(gq, "q4_k", gate, up, E, N, K, ids, x_t, "silu", "f32")
    h2, _ = run_glu_id(gq, "q4_k", gate, up, E, N, K, ids, x_t, "silu", "f32")
    h1 = h1.cpu().numpy()
    assert np.array_equal(h1.view(np.uint32), h2.cpu().numpy().view(np.uint32))
    ref, bound = glu_ref(orc, "q4_k", gate, up, E, N, K, ids, x, "silu", "f32")
    check(h1, ref, bound, "skewed")


def test_glu_id_bad_ids_counted_and_zero(gq, orc):
    g = synth.rng(0x67510009, 101)
    E, N, K, T, k = 8, 40, 512, 4, 3
    gate = synth.weight("q4_k", g, E * N, K)
    up = synth.weight("q4_k", g, E * N, K)
    ids = g.integers(0, E, (T, k)).astype(np.int32)
    ids[0, 1] = E
    ids[2, 0] = -1
    ids[3, 2] = 1 << 30
    x, x_t = make_x(g, (T, K), "f32")
    for hdt in ("f32", "bf16"):
        h, ws = run_glu_id(gq, "q4_k", gate, up, E, N, K, ids, x_t, "gelu_tanh", hdt)
        assert gq.gq_matvec_id_check(ws) == 3
        h = h.float().cpu().numpy()
        assert np.all(h[0, 1] == 0) and np.all(h[2, 0] == 0) and np.all(h[3, 2] == 0)
        ref, bound = glu_ref(orc, "q4_k", gate, up, E, N, K, ids, x, "gelu_tanh", hdt)
        check(h, ref, bound, "bad ids " + hdt)


def test_glu_id_edge_cases(gq):
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    ids = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    ws = torch.empty(gq.gq_matvec_id_workspace(3, 2, 2, 9), dtype=torch.uint8, device="cuda")
    # K == 0: every h row is act(0) * 0 = 0
    h = torch.full((2, 2, 9), float("nan"), device="cuda")
    gq.gq_matvec_id_glu("q4_0", e, e, 3, 9, 0, ids, torch.empty(2, 0, device="cuda"), "silu", h, ws)
    torch.cuda.synchronize()
    assert torch.all(h == 0)
    # no tokens, N == 0: no-ops that write nothing
    h2 = torch.full((1, 2, 4), 2.0, device="cuda")
    w = torch.empty(144 * 4, dtype=torch.uint8, device="cuda")
    gq.gq_matvec_id_glu("q4_k", w, w, 2, 4, 256, ids[:0], torch.zeros(0, 256, device="cuda"), "silu", h2, ws)
    gq.gq_matvec_id_glu("q4_k", w, w, 2, 0, 256, ids[:1], torch.zeros(1, 256, device="cuda"), "silu", h2[:, :, :0],
                        ws)
    torch.cuda.synchronize()
    assert torch.all(h2 == 2.0)
    need = gq.gq_matvec_id_workspace(2, 2, 2, 4)
    assert ws.numel() >= need
    w8 = torch.empty(144 * 8, dtype=torch.uint8, device="cuda")  # both experts' 4 rows
    with pytest.raises(gq.GqError, match="workspace"):
        gq.gq_matvec_id_glu("q4_k", w8, w8, 2, 4, 256, ids, torch.zeros(2, 256, device="cuda"), "silu", h,
                            ws[:need - 16])


@pytest.mark.parametrize("hdt", ["f32", "bf16"])
def test_moe_layer_route_glu_down(gq, orc, hdt):
    """128 experts, hidden 2816, expert FFN 704 (Q4_0); 8 tokens routed top-8
    on the device; gated unit (SiLU) in one launch; weighted down projection
    on its h.  Each step is checked against the oracle's step on the oracle's
    own inputs; the layer output against the oracle's layer."""
    E, H, F, T, k = 128, 2816, 704, 8, 8
    g = synth.rng(0x67510004, 0)
    logits = synth.router_logits(g, T, E)
    ids_t = torch.empty((T, k), dtype=torch.int32, device="cuda")
    rw_t = torch.empty((T, k), device="cuda")
    gq.gq_route_topk(dev(logits), k, ids_t, rw_t)
    ids, rw64 = orc.route_topk(logits, k)
    assert np.array_equal(ids_t.cpu().numpy(), ids)
    rw = rw_t.cpu().numpy()
    assert np.abs(rw - rw64).max() <= (k + 8) * 2.0 ** -24
    x = synth.normal_f32(g, (T, H))
    gate = synth.weight("q4_0", synth.rng(0x67510004, 1), E * F, H)
    up = synth.weight("q4_0", synth.rng(0x67510004, 2), E * F, H)
    down = synth.weight("q4_0", synth.rng(0x67510004, 3), E * H, F)

    ws = torch.empty(gq.gq_matvec_id_workspace(E, T, k, H), dtype=torch.uint8, device="cuda")
    h = torch.empty((T, k, F), device="cuda", dtype=torch.float32 if hdt == "f32" else torch.bfloat16)
    gq.gq_matvec_id_glu("q4_0", dev(gate), dev(up), E, F, H, ids_t, dev(x), "silu", h, ws)
    y = torch.full((T, H), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_0", dev(down), E, H, F, ids_t, h, True, y, ws, rw_t)
    torch.cuda.synchronize()

    h_ref, h_bound = glu_ref(orc, "q4_0", gate, up, E, F, H, ids, x, "silu", hdt)
    r = check(h.float().cpu().numpy(), h_ref, h_bound, "gated unit " + hdt)
    print("gated unit worst err/bound %.4f" % r)

    h32 = h_ref.astype(np.float32)
    y_ref, sa = orc.matvec_id("q4_0", down, E, H, F, ids, h32, True, rw)
    # the gated unit's error (and the fp32 rounding of the oracle's h) carried
    # through the down projection: sum_j |r_j| sum_k |w[n][k]| dh[t][j][k]
    dh = h_bound + np.abs(h_ref - h32)
    eb = H * F // QK["q4_0"] * BB["q4_0"]
    carry = np.zeros((T, H))
    for e in np.unique(ids):
        Wa = np.abs(orc.dequant("q4_0", down.reshape(-1)[e * eb:(e + 1) * eb]).astype(np.float64).reshape(H, F))
        for t_ in range(T):
            for j in range(k):
                if ids[t_, j] == e:
                    carry[t_] += abs(float(rw[t_, j])) * (Wa @ dh[t_, j])
    yv = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yv))
    err = np.abs(yv - y_ref)
    bound = 1e-3 * sa + carry
    assert not (err > bound).any(), "layer output: %d outside the bound" % (err > bound).sum()
    print("layer output worst err/bound %.4f" % float(np.max(err / bound)))


def test_glu_id_max_slots(gq, orc):
    """1024 slots (128 tokens, top 8), skewed so that runs span many groups."""
    g = synth.rng(0x67510009, 102)
    E, N, K, T, k = 48, 36, 512, 128, 8
    gate = synth.weight("q4_0", g, E * N, K)
    up = synth.weight("q4_0", g, E * N, K)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[::2, :4] = np.arange(4)
    x, x_t = make_x(g, (T, K), "bf16")
    h, ws = run_glu_id(gq, "q4_0", gate, up, E, N, K, ids, x_t, "silu", "bf16")
    ref, bound = glu_ref(orc, "q4_0", gate, up, E, N, K, ids, x, "silu", "bf16")
    check(h.float().cpu().numpy(), ref, bound, "S=1024")
    assert gq.gq_matvec_id_check(ws) == 0


@pytest.mark.parametrize("T", [8, 64])
def test_route_topk_plan_feeds_the_layer(gq, orc, T):
    """gq_route_topk_plan: ids and weights bit-identical to gq_route_topk's, and
    a table in ws that the gated unit and the weighted down projection use
    without ids, giving their results with ids bit for bit; the products of
    the tableless calls are also within the oracle's bounds."""
    E, H, F, k = 128, 2816, 704, 8
    g = synth.rng(0x67510004, 500 + T)
    logits = dev(synth.router_logits(g, T, E))
    ids_a = torch.empty((T, k), dtype=torch.int32, device="cuda")
    rw_a = torch.empty((T, k), device="cuda")
    gq.gq_route_topk(logits, k, ids_a, rw_a)
    ws = torch.empty(gq.gq_matvec_id_workspace(E, T, k, H), dtype=torch.uint8, device="cuda")
    ws.fill_(0xCD)
    ids_b = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    rw_b = torch.full((T, k), float("nan"), device="cuda")
    gq.gq_route_topk_plan(logits, k, ids_b, rw_b, ws)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b)
    assert torch.equal(rw_a.view(torch.int32), rw_b.view(torch.int32))
    x = dev(synth.normal_f32(g, (T, H)))
    gate = dev(synth.weight("q4_0", synth.rng(0x67510004, 1), E * F, H))
    up = dev(synth.weight("q4_0", synth.rng(0x67510004, 2), E * F, H))
    down = dev(synth.weight("q4_0", synth.rng(0x67510004, 3), E * H, F))
    # tableless calls on the routed table
    h = torch.full((T, k, F), float("nan"), device="cuda", dtype=torch.bfloat16)
    gq.gq_matvec_id_glu("q4_0", gate, up, E, F, H, (T, k), x, "silu", h, ws)
    y = torch.full((T, H), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_0", down, E, H, F, (T, k), h, True, y, ws, rw_b)
    yg = torch.full((T, k, F), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_0", gate, E, F, H, (T, k), x, False, yg, ws)
    # the same calls building their own tables
    ws2 = torch.empty_like(ws)
    h2 = torch.full((T, k, F), float("nan"), device="cuda", dtype=torch.bfloat16)
    gq.gq_matvec_id_glu("q4_0", gate, up, E, F, H, ids_a, x, "silu", h2, ws2)
    y2 = torch.full((T, H), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_0", down, E, H, F, ids_a, h2, True, y2, ws2, rw_a)
    yg2 = torch.full((T, k, F), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_0", gate, E, F, H, ids_a, x, False, yg2, ws2)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(yg.view(torch.int32), yg2.view(torch.int32))
    ids = ids_a.cpu().numpy()
    yref, sa = orc.matvec_id("q4_0", gate.cpu().numpy(), E, F, H, ids, x.cpu().numpy(), False)
    err = np.abs(yg.cpu().numpy().astype(np.float64) - yref)
    assert np.all(err <= 1e-3 * sa)


# (type, n_experts, hidden K, expert rows N, tokens, top_k, x dtype, h dtype, skew): the one-launch form at the
# MoE layer's shape, one token, experts taking more than 8 slots (two groups each), every format; then sizes
# that take the two launches (512 slots; more slots than experts)
ROUTED_GLU_CASES = [
    ("q4_0", 128, 2816, 704, 8, 8, "f32", "bf16", False),
    ("q4_0", 128, 2816, 704, 1, 8, "f32", "f32", False),
    ("q4_k", 64, 512, 256, 16, 4, "bf16", "bf16", True),
    ("q6_k", 64, 512, 256, 16, 4, "f32", "f32", True),
    ("q5_k", 100, 768, 256, 6, 6, "bf16", "f32", False),
    ("q4_0", 40, 256, 96, 5, 8, "f32", "bf16", True),
    ("q4_0", 128, 2816, 704, 64, 8, "f32", "bf16", False),
    ("q4_k", 16, 512, 256, 8, 4, "f32", "f32", False),
    ("q4_0", 64, 256, 64, 8, 8, "f32", "f32", "ties"),
]


@pytest.mark.parametrize("case", ROUTED_GLU_CASES, ids=lambda c: "%s_E%d_T%dk%d_%s%s" % (
    c[0], c[1], c[4], c[5], c[7], "_" + (c[8] if isinstance(c[8], str) else "skew") if c[8] else ""))
def test_route_matvec_id_glu_matches_routing_then_glu(gq, orc, case):
    """gq_route_matvec_id_glu: ids and weights bit-identical to gq_route_topk's
    and the oracle's ids; h bit-identical to gq_route_topk_plan then the
    tableless gq_matvec_id_glu, and within the oracle's bound; the table it
    leaves in ws gives the weighted down projection and an unweighted routed
    product bit for bit what the router's table gives them."""
    t, E, K, N, T, k, xdt, hdt, skew = case
    g = synth.rng(0x6751000B, E * 1000 + T * 10 + k)
    logits_np = synth.router_logits(g, T, E)
    if skew == "ties":  # logits on a coarse grid, with signed zeros: many equal logits (lower id first)
        logits_np = np.round(logits_np * 2.0).astype(np.float32) / np.float32(2.0)
        logits_np[logits_np == 0] = np.where(np.arange(int((logits_np == 0).sum())) % 2, -0.0, 0.0)
    elif skew:  # experts 3 and 5 chosen by every token: 2 groups each for 16 tokens
        logits_np[:, 3] += 50.0
        logits_np[:, 5] += 40.0
    logits = dev(logits_np)
    hdtype = torch.float32 if hdt == "f32" else torch.bfloat16
    x, x_t = make_x(g, (T, K), xdt)
    gate = synth.weight(t, synth.rng(0x6751000B, 1), E * N, K)
    up = synth.weight(t, synth.rng(0x6751000B, 2), E * N, K)
    down = synth.weight(t, synth.rng(0x6751000B, 3), E * K, N)
    gate_t, up_t, down_t = dev(gate), dev(up), dev(down)
    ws_n = max(N, K)

    def fresh():
        ws = torch.empty(gq.gq_matvec_id_workspace(E, T, k, ws_n), dtype=torch.uint8, device="cuda")
        ws.fill_(0xCD)  # contents need no initialisation
        return (ws, torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
                torch.full((T, k), float("nan"), device="cuda"),
                torch.full((T, k, N), float("nan"), device="cuda", dtype=hdtype))

    ws_a, ids_a, rw_a, h_a = fresh()  # one call
    gq.gq_route_matvec_id_glu(t, gate_t, up_t, E, N, K, logits, k, ids_a, rw_a, x_t, "silu", h_a, ws_a)
    ws_b, ids_b, rw_b, h_b = fresh()  # the router with its table, then the tableless gated unit
    gq.gq_route_topk_plan(logits, k, ids_b, rw_b, ws_b)
    gq.gq_matvec_id_glu(t, gate_t, up_t, E, N, K, (T, k), x_t, "silu", h_b, ws_b)
    ids_r = torch.empty((T, k), dtype=torch.int32, device="cuda")
    rw_r = torch.empty((T, k), device="cuda")
    gq.gq_route_topk(logits, k, ids_r, rw_r)
    outs = {}
    for name, ws, rw, h in (("a", ws_a, rw_a, h_a), ("b", ws_b, rw_b, h_b)):
        y = torch.full((T, K), float("nan"), device="cuda")
        gq.gq_matvec_id(t, down_t, E, K, N, (T, k), h, True, y, ws, rw)
        yg = torch.full((T, k, N), float("nan"), device="cuda")
        gq.gq_matvec_id(t, gate_t, E, N, K, (T, k), x_t, False, yg, ws)
        outs[name] = (y, yg)
    torch.cuda.synchronize()
    ids = ids_a.cpu().numpy()
    ids_o, _ = orc.route_topk(logits_np, k)
    assert np.array_equal(ids, ids_o)
    assert torch.equal(ids_a, ids_r) and torch.equal(ids_a, ids_b)
    assert torch.equal(rw_a.view(torch.int32), rw_r.view(torch.int32))
    assert torch.equal(rw_a.view(torch.int32), rw_b.view(torch.int32))
    hv = h_a.view(torch.int16) if hdt == "bf16" else h_a.view(torch.int32)
    assert torch.equal(hv, h_b.view(torch.int16) if hdt == "bf16" else h_b.view(torch.int32))
    for i in range(2):
        assert torch.equal(outs["a"][i].view(torch.int32), outs["b"][i].view(torch.int32)), ("y", "yg")[i]
    assert gq.gq_matvec_id_check(ws_a) == 0
    if skew is True:  # every token chose both (more than 8 slots each when T > 8)
        assert (ids == 3).sum() == T and (ids == 5).sum() == T
    ref, bound = glu_ref(orc, t, gate, up, E, N, K, ids, x, "silu", hdt)
    r = check(h_a.float().cpu().numpy(), ref, bound, "routed gated unit")
    print("routed gated unit worst err/bound %.4f" % r)
