"""GPU parity: gq_dequant and gq_matvec (through the C ABI) against the CPU
oracle on the same seeded inputs.

Bars: dequant bit-exact (fp32) and equal to the round-to-nearest-even of the
oracle's fp32 (bf16 / fp16); products within 1e-3 * sum_k |w_k x_k| per element
(and exactly zero where that sum is zero)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from block_quantized_weight_q4_amd import synth
from tests import packing

pytestmark = pytest.mark.gpu

TOL = 1e-3
TYPES = ("q4_0", "q4_k", "q6_k", "q5_k")


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


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_bound(y: np.ndarray, yref: np.ndarray, sumabs: np.ndarray, what: str = "") -> float:
    y = np.asarray(y, np.float64)
    assert y.shape == yref.shape
    assert np.all(np.isfinite(y)), "%s: non-finite output" % what
    err = np.abs(y - yref)
    bound = TOL * sumabs
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d elements outside 1e-3*sum|wx|; first at %s: y=%r ref=%r bound=%r" % (
            what, int(bad.sum()), bad.size, tuple(i), y[tuple(i)], yref[tuple(i)], bound[tuple(i)]))
    pos = bound > 0
    return float(np.max(err[pos] / bound[pos])) if pos.any() else 0.0


def make_x(g, B, K, xdt):
    x = synth.normal_f32(g, (B, K))
    if xdt == "bf16":
        bits = synth.bf16_bits(x)
        return synth.bf16_to_f32(bits), dev(bits.view(np.int16)).view(torch.bfloat16)
    return x, dev(x)


def run_matvec(gq, t, W_np, N, K, x_t, B):
    y = torch.full((B, N), float("nan"), device="cuda")
    gq.gq_matvec(t, dev(W_np), N, K, x_t, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ------------------------------------------------------------ dequant ----

def special_blocks(t: str, g) -> np.ndarray:
    """Blocks with zero, negative-zero, subnormal, negative and extreme fp16
    scales, and extreme integer fields."""
    specials = [0x0000, 0x8000, 0x0001, 0x03FF, 0x8001, 0x0400, 0x7BFF, 0xFBFF, 0xBC00, 0x3C00]
    out = []
    for i, s in enumerate(specials):
        b = synth.blocks(t, g, 1)[0].copy()
        if t == "q4_0":
            b[0], b[1] = s & 0xFF, s >> 8
        elif t in ("q4_k", "q5_k"):
            s2 = specials[(i + 3) % len(specials)]
            b[0], b[1], b[2], b[3] = s & 0xFF, s >> 8, s2 & 0xFF, s2 >> 8
            if i % 2:
                b[4:16] = 0xFF  # all scale/min bits set (63)
            if t == "q5_k" and i % 3 == 0:
                b[16:48] = 0xFF  # every fifth bit set
        else:
            b[208], b[209] = s & 0xFF, s >> 8
            if i % 3 == 0:
                b[192:208] = np.array([-128, 127, 0, -1] * 4, np.int8).view(np.uint8)
        out.append(b)
    return np.stack(out)


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_dequant_parity(gq, orc, t, odt):
    g = synth.rng(0x67510000, 100 + TYPES.index(t))
    blocks = np.concatenate([synth.blocks(t, g, 1537), special_blocks(t, g)])
    ref = orc.dequant(t, blocks)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[odt]
    out = torch.empty(ref.size, dtype=tdt, device="cuda")
    gq.gq_dequant(t, dev(blocks), out)
    torch.cuda.synchronize()
    if odt == "f32":
        got = out.cpu().numpy().view(np.uint32)
        assert np.array_equal(got, ref.view(np.uint32))
    elif odt == "bf16":
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, synth.bf16_bits(ref))
    else:
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        with np.errstate(over="ignore"):
            want = ref.astype(np.float16).view(np.uint16)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "%d mismatches, first: %s" % (bad.size, [
            (int(i), float(ref[i]), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]])


def test_dequant_empty_is_noop(gq):
    out = torch.full((8,), 7.0, device="cuda")
    gq.gq_dequant("q4_k", torch.empty(0, dtype=torch.uint8, device="cuda"), out[:0])
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# ------------------------------------------------------------- matvec ----

SHAPES = {
    "q4_0": [(1, 32), (3, 96), (705, 2048), (37, 2816), (64, 704), (257, 4096)],
    "q4_k": [(1, 256), (3, 512), (705, 2560), (130, 9728), (64, 17408), (9, 4096)],
    "q6_k": [(1, 256), (5, 512), (333, 5120), (70, 17408), (41, 1024)],
    "q5_k": [(1, 256), (3, 512), (705, 2560), (130, 9728), (9, 4096)],
}


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8])
def test_matvec_parity(gq, orc, t, xdt, B):
    worst = 0.0
    for si, (N, K) in enumerate(SHAPES[t]):
        g = synth.rng(0x67510000, 1000 * TYPES.index(t) + 10 * B + si)
        W = synth.weight(t, g, N, K)
        x, x_t = make_x(g, B, K, xdt)
        y = run_matvec(gq, t, W, N, K, x_t, B)
        yref, sa = orc.matvec(t, W, N, K, x)
        worst = max(worst, check_bound(y, yref, sa, "%s N=%d K=%d B=%d %s" % (t, N, K, B, xdt)))
    print("worst error / bound = %.4f" % worst)


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("B", [2, 4])
def test_matvec_batch_columns_bit_identical(gq, t, B):
    """Each column of a multi-vector dot-path product equals the batch-1
    product of that vector bit for bit (the dot-product path's multi-vector
    kernels agree with its one-vector kernel).  N > 4 K keeps batch 4 on the
    dot path."""
    N, K = (300, 4096) if t == "q4_0" else (300, 5120)
    if B == 4:
        N, K = (20000, 2048) if t == "q4_0" else (21000, 2560)
    g = synth.rng(0x67510000, 77)
    W = dev(synth.weight(t, g, N, K))
    for xdt in ("f32", "bf16"):
        x, x_t = make_x(g, B, K, xdt)
        y8 = torch.empty(B, N, device="cuda")
        gq.gq_matvec(t, W, N, K, x_t, y8)
        for b in range(B):
            y1 = torch.empty(1, N, device="cuda")
            gq.gq_matvec(t, W, N, K, x_t[b:b + 1].contiguous(), y1)
            torch.cuda.synchronize()
            assert torch.equal(y8[b].view(torch.int32), y1[0].view(torch.int32)), (xdt, b)


@pytest.mark.parametrize("t", TYPES)
def test_matvec_deterministic(gq, t):
    N, K = 1000, 2048 if t == "q4_0" else 2560
    g = synth.rng(0x67510000, 78)
    W = dev(synth.weight(t, g, N, K))
    _, x_t = make_x(g, 4, K, "f32")
    ys = []
    for _ in range(5):
        y = torch.empty(4, N, device="cuda")
        gq.gq_matvec(t, W, N, K, x_t, y)
        ys.append(y)
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int32), ys[0].view(torch.int32))


def test_matvec_edge_cases(gq, orc):
    g = synth.rng(0x67510000, 79)
    # K == 0 writes zeros; N == 0 leaves y alone
    y = torch.full((2, 5), float("nan"), device="cuda")
    gq.gq_matvec("q4_k", torch.empty(0, dtype=torch.uint8, device="cuda"), 5, 0,
                 torch.empty(2, 0, device="cuda"), y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
    y = torch.full((1, 4), 3.0, device="cuda")
    gq.gq_matvec("q4_k", torch.empty(16, dtype=torch.uint8, device="cuda"), 0, 256,
                 torch.zeros(1, 256, device="cuda"), y[:, :0])
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
    # weight matrix that starts 16 bytes into a larger buffer
    N, K = 33, 512
    W = synth.weight("q4_k", g, N, K)
    buf = np.zeros(W.size + 16, np.uint8)
    buf[16:] = W.reshape(-1)
    x = synth.normal_f32(g, (1, K))
    y = torch.empty(1, N, device="cuda")
    gq.gq_matvec("q4_k", dev(buf)[16:], N, K, dev(x), y)
    torch.cuda.synchronize()
    yref, sa = orc.matvec("q4_k", W, N, K, x)
    check_bound(y.cpu().numpy(), yref, sa, "offset W")


@pytest.mark.parametrize("t", TYPES)
def test_matvec_zero_point_rows_are_exactly_zero(gq, orc, t):
    """Rows whose quants all sit on the format's zero point (and Q4_K rows with
    zero scales and mins) have zero weights; their outputs must be exactly 0
    (the tolerance 1e-3 * sum|wx| is 0 there)."""
    g = synth.rng(0x67510000, 80)
    N, K = 12, 512
    W = synth.weight(t, g, N, K).copy()
    nb = K // (32 if t == "q4_0" else 256)
    bb = {"q4_0": 18, "q4_k": 144, "q6_k": 210, "q5_k": 176}[t]
    for r in range(0, N, 2):
        for j in range(nb):
            blk = W[r, j * bb:(j + 1) * bb]
            if t == "q4_0":
                blk[2:18] = 0x88
            elif t == "q6_k":
                blk[0:128] = 0x00
                blk[128:192] = 0xAA  # high parts 2 -> q = 32
            else:
                pack = packing.pack_q4_k if t == "q4_k" else packing.pack_q5_k
                blk[:] = pack(int(blk[0]) | int(blk[1]) << 8, int(blk[2]) | int(blk[3]) << 8,
                              [int(v) for v in g.integers(0, 64, 8)], [0] * 8, [0] * 256)
    x = synth.normal_f32(g, (3, K))
    y = run_matvec(gq, t, W, N, K, dev(x), 3)
    yref, sa = orc.matvec(t, W, N, K, x)
    assert np.all(yref[:, ::2] == 0) and np.all(sa[:, ::2] == 0)
    assert np.all(y[:, ::2] == 0)
    check_bound(y, yref, sa, t)


@pytest.mark.parametrize("t", TYPES)
def test_matvec_wide_dynamic_range(gq, orc, t):
    """Activations spanning 16 decades (each element scaled by 10^U(-8, 8));
    the per-32 power-of-two scaling keeps the fp16 activations in range."""
    g = synth.rng(0x67510000, 81)
    N, K = 64, 1024
    W = synth.weight(t, g, N, K)
    x = (synth.normal_f32(g, (2, K)) * 10.0 ** g.uniform(-8, 8, (2, K))).astype(np.float32)
    x[1] *= np.float32(1e-30)  # tiny overall scale
    y = run_matvec(gq, t, W, N, K, dev(x), 2)
    yref, sa = orc.matvec(t, W, N, K, x)
    check_bound(y, yref, sa, t)


def test_matvec_nan_propagates(gq):
    g = synth.rng(0x67510000, 82)
    N, K = 40, 512
    W = dev(synth.weight("q4_k", g, N, K))
    x = synth.normal_f32(g, (2, K))
    x[1, 300] = np.nan
    y = torch.empty(2, N, device="cuda")
    gq.gq_matvec("q4_k", W, N, K, dev(x), y)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.all(np.isfinite(y[0])) and np.all(np.isnan(y[1]))


# ------------------------------------------------ full-size workloads ----

def dense_layer_shapes(hidden=2560):
    # (name, N, K): q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up 9728x2560, down 2560x9728
    return [("q", 4096, hidden), ("k", 1024, hidden), ("v", 1024, hidden), ("o", hidden, 4096),
            ("gate", 9728, hidden), ("up", 9728, hidden), ("down", hidden, 9728)]


def mixed_layer_shapes():
    # hidden 5120, FFN 17408: gate/up/q/o/k Q4_K, down/v Q6_K
    return [("q", "q4_k", 5120, 5120), ("k", "q4_k", 1024, 5120), ("v", "q6_k", 1024, 5120),
            ("o", "q4_k", 5120, 5120), ("gate", "q4_k", 17408, 5120), ("up", "q4_k", 17408, 5120),
            ("down", "q6_k", 5120, 17408)]


def test_workload_q4_0_2048(gq, orc):
    g = synth.rng(0x67510001, 0)
    N = K = 2048
    W = synth.weight("q4_0", g, N, K)
    x = synth.normal_f32(g, (1, K))
    y = run_matvec(gq, "q4_0", W, N, K, dev(x), 1)
    yref, sa = orc.matvec("q4_0", W, N, K, x)
    r = check_bound(y, yref, sa, "Q4_0 2048x2048")
    print("Q4_0 2048x2048 worst err/bound %.4f" % r)


@pytest.mark.parametrize("B", [1, 4])
def test_workload_q4_k_dense_layer(gq, orc, B):
    for i, (name, N, K) in enumerate(dense_layer_shapes()):
        g = synth.rng(0x67510002, i)
        W = synth.weight("q4_k", g, N, K)
        x = synth.normal_f32(synth.rng(0x67510002, 100 + 10 * B + i), (B, K))
        y = run_matvec(gq, "q4_k", W, N, K, dev(x), B)
        yref, sa = orc.matvec("q4_k", W, N, K, x)
        r = check_bound(y, yref, sa, "%s B=%d" % (name, B))
        print("%s %dx%d B=%d worst err/bound %.4f" % (name, N, K, B, r))


@pytest.mark.parametrize("B", [1, 2, 8])
def test_workload_mixed_layer_bf16(gq, orc, B):
    for i, (name, t, N, K) in enumerate(mixed_layer_shapes()):
        g = synth.rng(0x67510003, i)
        W = synth.weight(t, g, N, K)
        x, x_t = make_x(synth.rng(0x67510003, 100 + 10 * B + i), B, K, "bf16")
        y = run_matvec(gq, t, W, N, K, x_t, B)
        yref, sa = orc.matvec(t, W, N, K, x)
        r = check_bound(y, yref, sa, "%s %s B=%d" % (name, t, B))
        print("%s %s %dx%d B=%d worst err/bound %.4f" % (name, t, N, K, B, r))
