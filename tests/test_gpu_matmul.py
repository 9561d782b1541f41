"""GPU parity of gq_matmul (Q4_0 / Q4_K / Q6_K x bf16 prefill product on the
matrix cores) against the CPU oracle.

Bar: |Y - Y_ref| <= 1e-3 * sum_k |X w| per element (weights enter the matrix
cores as bf16, the rounding that the prefill reading fixes; Y_ref uses the exact
fp32 weights).  Small shapes are compared element by element; the full
3015 x 17408 x 5120 Q4_K workload (and the Q6_K down projection of the same
layer family, 3015 x 5120 x 17408) on sampled full rows and columns plus a
Freivalds checksum of the whole output."""
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


def check_bound(y, yref, sumabs, what=""):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), what
    err = np.abs(y - yref)
    bound = 1e-3 * sumabs
    bad = err > bound
    assert not bad.any(), "%s: %d elements outside the bound, first %s (y=%r ref=%r)" % (
        what, bad.sum(), np.argwhere(bad)[0], y[tuple(np.argwhere(bad)[0])], yref[tuple(np.argwhere(bad)[0])])
    pos = bound > 0
    return float(np.max(err[pos] / bound[pos])) if pos.any() else 0.0


def make_X(g, M, K, ldx=None):
    ldx = ldx or K
    x = synth.normal_f32(g, (M, K))
    bits = synth.bf16_bits(x)
    buf = np.zeros((M, ldx), np.uint16)
    buf[:, :K] = bits
    return synth.bf16_to_f32(bits), dev(buf.view(np.int16)).view(torch.bfloat16)


# The 1e-3 * sum|Xw| bar is met statistically: each weight carries a bf16
# rounding (2^-9 relative) and the errors average over K, so it is asserted
# for K >= 1024 (the workload has K = 5120); test_matmul_is_bf16_weight_product
# checks the arithmetic itself at any K.
SMALL = [(1, 64, 1024, 0, 0), (37, 130, 1024, 8, 6), (256, 128, 2048, 0, 0), (300, 257, 1024, 0, 3),
         (513, 200, 1536, 64, 12), (7, 1000, 2048, 0, 0), (12, 40, 5120, 0, 0)]
# Q4_0 rows may end half way into a 64-input stage (K = 32 mod 64)
SMALL_Q4_0 = [(1, 64, 1056, 0, 0), (37, 130, 1024, 8, 6), (300, 257, 2080, 0, 3), (513, 200, 1536, 64, 12),
              (7, 1000, 2048, 0, 0)]


@pytest.mark.parametrize("t,M,N,K,padx,pady", [("q4_k",) + c for c in SMALL] + [("q6_k",) + c for c in SMALL]
                         + [("q4_0",) + c for c in SMALL_Q4_0] + [("q5_k",) + c for c in SMALL[:4]])
def test_matmul_small_full_compare(gq, orc, t, M, N, K, padx, pady):
    g = synth.rng(0x67510005, M * 7 + N + 100000 * ("q4_k", "q6_k", "q4_0", "q5_k").index(t))
    W = synth.weight(t, g, N, K)
    xf, X = make_X(g, M, K, K + padx)
    Y = torch.full((M, N + pady), float("nan"), device="cuda")
    gq.gq_matmul(t, dev(W), N, K, X, Y)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    yref, sa = orc.matmul_rows(t, W, N, K, xf, np.arange(M))
    r = check_bound(y[:, :N], yref, sa, "%s M=%d N=%d K=%d" % (t, M, N, K))
    if pady:
        assert np.all(np.isnan(y[:, N:])), "padding columns of Y were written"
    print("worst err/bound %.4f" % r)


@pytest.mark.parametrize("t,M,N,K", [("q4_k", 1, 64, 256), ("q4_k", 37, 132, 512), ("q4_k", 256, 128, 256),
                                     ("q4_k", 300, 260, 768), ("q6_k", 1, 64, 256), ("q6_k", 37, 132, 512),
                                     ("q6_k", 300, 260, 768), ("q4_0", 1, 64, 32), ("q4_0", 37, 132, 96),
                                     ("q4_0", 256, 128, 64), ("q4_0", 300, 260, 544), ("q5_k", 37, 132, 512),
                                     ("q5_k", 300, 260, 768)])
def test_matmul_is_bf16_weight_product(gq, orc, t, M, N, K):
    """The kernel computes sum_k X[m][k] * bf16(w[n][k]) with w the exact fp32
    weight (oracle dequant) rounded to nearest even: compared with an fp64
    product of those rounded weights, within an fp32 accumulation bound."""
    g = synth.rng(0x67510005, 500 + M + 1000 * ("q4_k", "q6_k", "q4_0", "q5_k").index(t))
    W = synth.weight(t, g, N, K)
    xf, X = make_X(g, M, K)
    Y = torch.empty((M, N), device="cuda")
    gq.gq_matmul(t, dev(W), N, K, X, Y)
    torch.cuda.synchronize()
    wb = synth.bf16_to_f32(synth.bf16_bits(orc.dequant(t, W))).reshape(N, K).astype(np.float64)
    ref = xf.astype(np.float64) @ wb.T
    absref = np.abs(xf.astype(np.float64)) @ np.abs(wb).T
    err = np.abs(Y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= K * 2.0 ** -23 * absref), float(np.max(err / np.maximum(absref, 1e-30)))


def test_matmul_empty_is_noop(gq):
    Y = torch.full((4, 8), 5.0, device="cuda")
    gq.gq_matmul("q4_k", torch.empty(8 * 144, dtype=torch.uint8, device="cuda"), 8, 256,
                 torch.empty(0, 256, dtype=torch.bfloat16, device="cuda"), Y[:0])
    torch.cuda.synchronize()
    assert torch.all(Y == 5.0)


# The full-size prefill products (every launch bench.py times) are checked in
# tests/test_gpu_timed_launches.py: NaN-filled Y, 64 sampled rows, columns and
# two checksums.


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q4_0"])
def test_matmul_tail_round_split_along_k(gq, orc, t):
    """4000 x 4352 outputs = 16 x 17 tiles of 256: on 256 CUs the last 16
    tiles form a short last round, which the kernel runs as two K halves added
    into zeroed output.  Sampled rows of the last (partial) row of tiles and
    columns of the split tiles are compared in full; a second call gives the
    same bits."""
    M, N, K = 4000, 4352, 1024
    g = synth.rng(0x67510005, 700 + ("q4_k", "q6_k", "q4_0").index(t))
    W = synth.weight(t, g, N, K)
    xf, X = make_X(g, M, K)
    Wd = dev(W)
    Y = torch.full((M, N), float("nan"), device="cuda")
    gq.gq_matmul(t, Wd, N, K, X, Y)
    Y2 = torch.full((M, N), float("nan"), device="cuda")
    gq.gq_matmul(t, Wd, N, K, X, Y2)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y).all())
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
    s = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, 3840, M - 1], s.choice(np.arange(3841, M - 1), 12, replace=False),
                                     s.choice(np.arange(1, 3840), 6, replace=False)]))
    cols = np.unique(np.concatenate([[0, 255, 256, N - 1], s.choice(np.arange(257, N - 1), 8, replace=False)]))
    ref, sa = orc.matmul_rows(t, W, N, K, xf, rows)
    check_bound(Y[torch.from_numpy(rows).cuda()].cpu().numpy(), ref, sa, "rows")
    refc, sac = orc.matmul_cols(t, W, N, K, xf, cols)
    check_bound(Y[:, torch.from_numpy(cols).cuda()].cpu().numpy(), refc, sac, "cols")


@pytest.mark.parametrize("t,rem,K", [("q4_k", 100, 1024), ("q4_k", 200, 1024), ("q5_k", 100, 1024),
                                     ("q4_0", 200, 1056), ("q6_k", 100, 1024)])
def test_matmul_last_round_in_quarters(gq, orc, t, rem, K):
    """M = 300 rows (two rows of tiles) and N chosen so that the tile count is
    the CU count plus 4: the last round holds 4 tiles, which the 8-wavefront
    kernel runs as N and K quarters (Q6_K as K halves).  The last column of
    tiles is rem < 256 wide, so its second N quarter is empty (rem <= 128) or
    partial.  Y is NaN-filled: every output must be written; two calls give
    the same bits; sampled rows and columns of the last tiles against the
    oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert cus % 2 == 0, cus
    M, gn = 300, cus // 2 + 2
    N = (gn - 1) * 256 + rem
    g = synth.rng(0x67510005, 900 + rem + K + ("q4_k", "q6_k", "q4_0", "q5_k").index(t))
    W = synth.weight(t, g, N, K)
    xf, X = make_X(g, M, K)
    Wd = dev(W)
    Y = torch.full((M, N), float("nan"), device="cuda")
    gq.gq_matmul(t, Wd, N, K, X, Y)
    Y2 = torch.full((M, N), float("nan"), device="cuda")
    gq.gq_matmul(t, Wd, N, K, X, Y2)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y).all())
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
    s = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], s.choice(np.arange(257, M - 1), 8, replace=False)]))
    last = (gn - 4) * 256  # first column of the last round's tiles
    cols = np.unique(np.concatenate([[0, last - 1, last, N - 1, N - rem, N - rem + 127],
                                     s.choice(np.arange(last + 1, N - 1), 10, replace=False)]))
    cols = cols[cols < N]
    ref, sa = orc.matmul_rows(t, W, N, K, xf, rows)
    check_bound(Y[torch.from_numpy(rows).cuda()].cpu().numpy(), ref, sa, "rows")
    refc, sac = orc.matmul_cols(t, W, N, K, xf, cols)
    check_bound(Y[:, torch.from_numpy(cols).cuda()].cpu().numpy(), refc, sac, "cols")
