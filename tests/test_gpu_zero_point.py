"""GPU parity where almost every quant sits on its format's zero point.

Rows whose weights are all zero except one per 32-weight group make
sum_k |w_k x_k| tiny, so the bar 1e-3 * sum|w x| leaves no room for a sum that
carries the zero point (or any other offset) through its fp32 accumulation:
each product must reach the accumulator as (q - z) * x, with nothing that
cancels only later.  The activation at the one non-zero weight is made small
next to the rest of its 32-group, which also checks that the per-group
activation scaling keeps small elements exact enough.

Both decode paths are covered: the dot-product path (1-4 vectors) and the
matrix-core path (8 and 16 vectors); fp32 and bf16 activations; all four block
types (Q4_0 q = 8, Q6_K q = 32, Q4_K / Q5_K with zero mins and q = 0)."""
from __future__ import annotations

import numpy as np
import pytest

from block_quantized_weight_q4_amd import synth
from tests import packing
from tests.test_gpu_dequant_matvec import TYPES, _name_the_case, check_bound, dev, gq, make_x, run_matvec  # noqa: F401

pytestmark = pytest.mark.gpu


def near_zero_point_weight(t: str, g, N: int, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Packed [N][row bytes] weights whose quants all equal the zero point
    except one per 32-weight group, and the [N][K] mask of those positions."""
    qk, bb = synth.BLOCK[t]
    nb = K // qk
    W = np.empty((N, nb * bb), np.uint8)
    off = np.zeros((N, K), bool)
    for r in range(N):
        for j in range(nb):
            zp = {"q4_0": 8, "q6_k": 32}.get(t, 0)
            q = [zp] * qk
            for grp in range(qk // 32):
                i = 32 * grp + int(g.integers(0, 32))
                hi = {"q4_0": 16, "q6_k": 64, "q4_k": 16, "q5_k": 32}[t]
                v = int(g.integers(0, hi - 1))
                q[i] = v if v < zp else v + 1  # any value but the zero point
                off[r, j * qk + i] = True
            d = packing.f16_bits(float(abs(g.standard_normal())) * 0.01 + 1e-4)
            if t == "q4_0":
                blk = packing.pack_q4_0(d, q)
            elif t == "q6_k":
                sc = [int(v) for v in g.integers(1, 128, 16) * g.choice([-1, 1], 16)]
                blk = packing.pack_q6_k(d, sc, q)
            else:
                pack = packing.pack_q4_k if t == "q4_k" else packing.pack_q5_k
                dmin = packing.f16_bits(float(abs(g.standard_normal())) * 1e-3)
                blk = pack(d, dmin, [int(v) for v in g.integers(1, 64, 8)], [0] * 8, q)
            W[r, j * bb:(j + 1) * bb] = blk
    return W, off


def shrink_at(x: np.ndarray, off: np.ndarray, rows) -> np.ndarray:
    """x with the activations at the non-zero weights of the given rows scaled
    by 2^-10 (all rows share x, so the union of their positions)."""
    x = x.copy()
    mask = off[rows].any(axis=0)
    x[:, mask] *= np.float32(2.0 ** -10)
    return x


CASES = [  # (N, K) per type; the dot path gets B <= 4, the matrix cores 8 and 16
    ("q4_0", 48, 2048), ("q4_k", 48, 2560), ("q5_k", 32, 2560), ("q6_k", 40, 2560),
]


@pytest.mark.parametrize("t,N,K", CASES)
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("B", [1, 2, 8, 16])
def test_matvec_near_zero_point(gq, orc, t, N, K, xdt, B):
    g = synth.rng(0x67510000, 300 + 10 * TYPES.index(t) + B)
    W, off = near_zero_point_weight(t, g, N, K)
    x, _ = make_x(g, B, K, xdt)
    x = shrink_at(x, off, slice(0, N // 2))
    if xdt == "bf16":
        bits = synth.bf16_bits(x)
        x = synth.bf16_to_f32(bits)
        import torch
        x_t = dev(bits.view(np.int16)).view(torch.bfloat16)
    else:
        x_t = dev(x)
    y = run_matvec(gq, t, W, N, K, x_t, B)
    yref, sa = orc.matvec(t, W, N, K, x)
    r = check_bound(y, yref, sa, "%s N=%d K=%d B=%d %s" % (t, N, K, B, xdt))
    print("worst err/bound %.4f" % r)


@pytest.mark.parametrize("t", ["q4_0", "q4_k", "q5_k", "q6_k"])
def test_matvec_near_zero_point_batch4_dot_path(gq, orc, t):
    """Four vectors on a matrix with many short rows (N > 4 K keeps batch 4 on
    the dot-product path for every type)."""
    N, K = (2100, 512) if t != "q4_0" else (2100, 256)
    g = synth.rng(0x67510000, 350 + TYPES.index(t))
    W, off = near_zero_point_weight(t, g, N, K)
    x, x_t = make_x(g, 4, K, "f32")
    x = shrink_at(x, off, slice(0, 8))
    y = run_matvec(gq, t, W, N, K, dev(x), 4)
    yref, sa = orc.matvec(t, W, N, K, x)
    check_bound(y, yref, sa, "%s B=4 dot path" % t)
