"""GPU parity of gq_matvec_id (routed experts) against the CPU oracle.

Bars: per-slot outputs within 1e-3 * sum_k |w x|; routing-weighted outputs
within 1e-3 * sum_j |r_j| * sum_k |w x|; invariants that reduce the routed
product to gq_matvec bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from block_quantized_weight_q4_amd import synth

pytestmark = pytest.mark.gpu

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


def check_bound(y, yref, sumabs, what=""):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), what
    err = np.abs(y - yref)
    bound = 1e-3 * sumabs
    bad = err > bound
    assert not bad.any(), "%s: %d elements outside the bound, first %s" % (what, bad.sum(), np.argwhere(bad)[0])
    pos = bound > 0
    return float(np.max(err[pos] / bound[pos])) if pos.any() else 0.0


def run_id(gq, t, experts_np, E, N, K, ids_np, x_t, per_slot, route_w=None):
    T, k = ids_np.shape
    ws = torch.empty(gq.gq_matvec_id_workspace(E, T, k, N), dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)  # contents need no initialisation
    shape = (T, N) if route_w is not None else (T, k, N)
    y = torch.full(shape, float("nan"), device="cuda")
    gq.gq_matvec_id(t, dev(experts_np), E, N, K, dev(ids_np), x_t, per_slot, y, ws,
                    None if route_w is None else dev(route_w))
    torch.cuda.synchronize()
    return y.cpu().numpy(), ws


def test_moe_workload_gate_up_down(gq, orc):
    """128 experts, hidden 2816, expert FFN 704 (Q4_0); 8 tokens routed top-8
    on the device (gq_route_topk over seeded logits), softmax weights on the
    down projection.  The oracle products take the oracle's own routing, which
    the device's ids match bit for bit."""
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
    print("distinct experts:", len(np.unique(ids)))
    x = synth.normal_f32(g, (T, H))
    for name, N, K in (("gate", F, H), ("up", F, H)):
        ex = synth.weight("q4_0", synth.rng(0x67510004, 1 + (name == "up")), E * N, K)
        y, ws = run_id(gq, "q4_0", ex, E, N, K, ids, dev(x), False)
        yref, sa = orc.matvec_id("q4_0", ex, E, N, K, ids, x, False)
        r = check_bound(y, yref, sa, name)
        print("%s worst err/bound %.4f" % (name, r))
        assert gq.gq_matvec_id_check(ws) == 0
    h = synth.normal_f32(g, (T, k, F))
    exd = synth.weight("q4_0", synth.rng(0x67510004, 3), E * H, F)
    y, ws = run_id(gq, "q4_0", exd, E, H, F, ids, dev(h), True, rw)
    yref, sa = orc.matvec_id("q4_0", exd, E, H, F, ids, h, True, rw)
    r = check_bound(y, yref, sa, "down")
    print("down (routed) worst err/bound %.4f" % r)


@pytest.mark.parametrize("t", ["q4_0", "q4_k", "q6_k", "q5_k"])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_matvec_id_shapes(gq, orc, t, xdt):
    g = synth.rng(0x67510004, 10 + ["q4_0", "q4_k", "q6_k", "q5_k"].index(t))
    for (E, N, K, T, k) in ((5, 37, 512, 3, 2), (16, 130, 1024, 6, 4), (9, 64, 2048, 16, 3)):
        ex = synth.weight(t, g, E * N, K)
        ids = g.integers(0, E, (T, k)).astype(np.int32)
        for per_slot in (False, True):
            x = synth.normal_f32(g, (T, k, K) if per_slot else (T, K))
            if xdt == "bf16":
                bits = synth.bf16_bits(x)
                x = synth.bf16_to_f32(bits)
                x_t = dev(bits.view(np.int16)).view(torch.bfloat16)
            else:
                x_t = dev(x)
            y, _ = run_id(gq, t, ex, E, N, K, ids, x_t, per_slot)
            yref, sa = orc.matvec_id(t, ex, E, N, K, ids, x, per_slot)
            check_bound(y, yref, sa, "%s E=%d N=%d K=%d per_slot=%s" % (t, E, N, K, per_slot))
            rw = g.random((T, k)).astype(np.float32)
            y, _ = run_id(gq, t, ex, E, N, K, ids, x_t, per_slot, rw)
            yref, sa = orc.matvec_id(t, ex, E, N, K, ids, x, per_slot, rw)
            check_bound(y, yref, sa, "%s routed" % t)


@pytest.mark.parametrize("t", ["q4_0", "q4_k"])
def test_matvec_id_single_expert_equals_matvec(gq, t):
    """Every slot routed to one expert (groups of up to 8 slots, two groups):
    each output row equals gq_matvec of that expert on the same vector, bit for
    bit (at this size both launches take the same lanes per row, which fixes
    the summation order)."""
    g = synth.rng(0x67510004, 20)
    E, N, K, T, k = 6, 96, 1024, 7, 2
    ex = synth.weight(t, g, E * N, K)
    ids = np.full((T, k), 3, np.int32)
    x = synth.normal_f32(g, (T, K))
    y, _ = run_id(gq, t, ex, E, N, K, ids, dev(x), False)
    eb = N * K // QK[t] * BB[t]
    W3 = dev(ex.reshape(-1)[3 * eb:4 * eb])
    # gq_matvec with 1 or 2 vectors runs the dot-product path, whose columns
    # match its 4-vector kernel's bit for bit
    for tok0 in range(0, T, 2):
        xs = x[tok0:tok0 + 2]
        yy = torch.empty(xs.shape[0], N, device="cuda")
        gq.gq_matvec(t, W3, N, K, dev(xs), yy)
        torch.cuda.synchronize()
        yy = yy.cpu().numpy()
        for i in range(xs.shape[0]):
            for j in range(k):
                assert np.array_equal(y[tok0 + i, j].view(np.uint32), yy[i].view(np.uint32))


def test_matvec_id_bad_ids_counted_and_zero(gq, orc):
    g = synth.rng(0x67510004, 21)
    E, N, K, T, k = 8, 40, 512, 4, 3
    ex = synth.weight("q4_k", g, E * N, K)
    ids = g.integers(0, E, (T, k)).astype(np.int32)
    ids[0, 1] = E        # one past the end
    ids[2, 0] = -1       # negative
    ids[3, 2] = 1 << 30  # far out
    x = synth.normal_f32(g, (T, K))
    y, ws = run_id(gq, "q4_k", ex, E, N, K, ids, dev(x), False)
    assert gq.gq_matvec_id_check(ws) == 3
    yref, sa = orc.matvec_id("q4_k", ex, E, N, K, ids, x, False)
    assert np.all(y[0, 1] == 0) and np.all(y[2, 0] == 0) and np.all(y[3, 2] == 0)
    check_bound(y, yref, sa, "bad ids")
    rw = g.random((T, k)).astype(np.float32)
    y, ws = run_id(gq, "q4_k", ex, E, N, K, ids, dev(x), False, rw)
    yref, sa = orc.matvec_id("q4_k", ex, E, N, K, ids, x, False, rw)
    check_bound(y, yref, sa, "bad ids routed")
    assert gq.gq_matvec_id_check(ws) == 3


def test_matvec_id_many_slots_one_expert_and_determinism(gq, orc):
    """256 slots, heavily skewed routing (most to two experts): long runs split
    into many groups; repeated calls are bit-identical."""
    g = synth.rng(0x67510004, 22)
    E, N, K, T, k = 32, 72, 768, 64, 4
    ex = synth.weight("q4_k", g, E * N, K)
    ids = np.where(g.random((T, k)) < 0.7, g.integers(0, 2, (T, k)), g.integers(0, E, (T, k))).astype(np.int32)
    x = synth.normal_f32(g, (T, K))
    rw = g.random((T, k)).astype(np.float32)
    y1, _ = run_id(gq, "q4_k", ex, E, N, K, ids, dev(x), False, rw)
    y2, _ = run_id(gq, "q4_k", ex, E, N, K, ids, dev(x), False, rw)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    yref, sa = orc.matvec_id("q4_k", ex, E, N, K, ids, x, False, rw)
    check_bound(y1, yref, sa, "skewed")


@pytest.mark.parametrize("E", [64, 1500])
def test_matvec_id_max_slots_and_many_experts(gq, orc, E):
    """1024 slots (128 tokens, top 8; the largest call) and, with 1500 experts,
    the group table built without the per-expert histogram."""
    g = synth.rng(0x67510004, 30 + E)
    N, K, T, k = 40, 256, 128, 8
    if E > 1024:
        T, k = 24, 6
    ex = synth.weight("q4_k", g, E * N, K)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if E <= 1024:
        ids[::3] = ids[0]  # many tokens on the same experts: long runs split into groups
    x = synth.normal_f32(g, (T, K))
    y, ws = run_id(gq, "q4_k", ex, E, N, K, ids, dev(x), False)
    yref, sa = orc.matvec_id("q4_k", ex, E, N, K, ids, x, False)
    check_bound(y, yref, sa, "E=%d S=%d per slot" % (E, T * k))
    assert gq.gq_matvec_id_check(ws) == 0
    rw = g.random((T, k)).astype(np.float32)
    y, _ = run_id(gq, "q4_k", ex, E, N, K, ids, dev(x), False, rw)
    yref, sa = orc.matvec_id("q4_k", ex, E, N, K, ids, x, False, rw)
    check_bound(y, yref, sa, "E=%d S=%d routed" % (E, T * k))


def test_matvec_id_reused_table(gq, orc):
    """A weighted product called without ids uses the group table the
    previous routed call left in the same workspace (invalid ids included):
    its result equals a call that builds the table itself, bit for bit, and the
    invalid-id count is still the table's."""
    g = synth.rng(0x67510004, 40)
    E, N, K, T, k = 12, 48, 512, 5, 3
    ex = synth.weight("q4_k", g, E * N, K)
    exd = synth.weight("q4_k", g, E * K, 512)  # down-like: K rows of 512 inputs per expert
    ids = g.integers(0, E, (T, k)).astype(np.int32)
    ids[1, 2] = E + 5
    x = synth.normal_f32(g, (T, K))
    h = synth.normal_f32(g, (T, k, 512))
    rw = g.random((T, k)).astype(np.float32)
    ids_t, rw_t = dev(ids), dev(rw)
    ws = torch.empty(max(gq.gq_matvec_id_workspace(E, T, k, N), gq.gq_matvec_id_workspace(E, T, k, K)),
                     dtype=torch.uint8, device="cuda")
    y0 = torch.full((T, k, N), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_k", dev(ex), E, N, K, ids_t, dev(x), False, y0, ws)  # builds the table
    yr = torch.full((T, K), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_k", dev(exd), E, K, 512, (T, k), dev(h), True, yr, ws, rw_t)  # reuses it
    torch.cuda.synchronize()
    assert gq.gq_matvec_id_check(ws) == 1
    yf = torch.full((T, K), float("nan"), device="cuda")
    gq.gq_matvec_id("q4_k", dev(exd), E, K, 512, ids_t, dev(h), True, yf, ws, rw_t)
    torch.cuda.synchronize()
    assert torch.equal(yr.view(torch.int32), yf.view(torch.int32))
    yref, sa = orc.matvec_id("q4_k", exd, E, K, 512, ids, h, True, rw)
    check_bound(yr.cpu().numpy(), yref, sa, "reused table")


def test_moe_64_tokens_top8(gq, orc):
    """The routed-expert shapes (128 Q4_0 experts, hidden 2816, FFN 704) at 64
    tokens routed top-8 on the device: 512 slots, about 4 per expert, so
    several experts receive more than the 4 slots one group held before; every
    expert is read once per group of up to 8 of its slots (the printed count of
    expert reads against the distinct experts)."""
    E, H, F, T, k = 128, 2816, 704, 64, 8
    g = synth.rng(0x67510004, 64)
    logits = synth.router_logits(g, T, E)
    ids_t = torch.empty((T, k), dtype=torch.int32, device="cuda")
    rw_t = torch.empty((T, k), device="cuda")
    gq.gq_route_topk(dev(logits), k, ids_t, rw_t)
    torch.cuda.synchronize()
    ids, _ = orc.route_topk(logits, k)
    assert np.array_equal(ids_t.cpu().numpy(), ids)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    reads = int(np.sum((counts + 7) // 8))
    print("distinct experts %d, max slots per expert %d, expert reads %d (groups of 4 would read %d)"
          % (int(np.sum(counts > 0)), int(counts.max()), reads, int(np.sum((counts + 3) // 4))))
    x = synth.normal_f32(g, (T, H))
    gate = synth.weight("q4_0", synth.rng(0x67510004, 1), E * F, H)
    y, ws = run_id(gq, "q4_0", gate, E, F, H, ids, dev(x), False)
    yref, sa = orc.matvec_id("q4_0", gate, E, F, H, ids, x, False)
    check_bound(y, yref, sa, "gate, 64 tokens")
    rw = rw_t.cpu().numpy()
    h = synth.normal_f32(g, (T, k, F))
    down = synth.weight("q4_0", synth.rng(0x67510004, 3), E * H, F)
    y, _ = run_id(gq, "q4_0", down, E, H, F, ids, dev(h), True, rw)
    yref, sa = orc.matvec_id("q4_0", down, E, H, F, ids, h, True, rw)
    check_bound(y, yref, sa, "down, 64 tokens")
