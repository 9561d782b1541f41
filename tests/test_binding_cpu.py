"""The Python binding rejects mistaken arguments before it calls the library.

The C ABI receives bare pointers, so a tensor of the wrong element type, too
few elements, a non-unit stride or host memory would turn into an
out-of-bounds device access.  Every such case must raise here, on the host,
without a GPU: the binding checks element types first, then sizes and layout,
then the device, so host tensors of the right size and type reach the last
check (TypeError "must be a GPU tensor") and anything wrong before that raises
its own error.  No test here launches anything."""
from __future__ import annotations

import pytest
import torch

gq = pytest.importorskip("block_quantized_weight_q4_amd._binding")

f32, bf16, u8, i32 = torch.float32, torch.bfloat16, torch.uint8, torch.int32
RB = {"q4_0": 18 * 2048 // 32, "q4_k": 144 * 2560 // 256}  # row bytes at K = 2048 / 2560


def host(*shape, dtype=f32):
    return torch.zeros(*shape, dtype=dtype)


def raises_gpu(fn, *a, **k):
    with pytest.raises(TypeError, match="GPU tensor"):
        fn(*a, **k)


def test_matvec_checks():
    N, K = 64, 2560
    W, x, y = host(N * RB["q4_k"], dtype=u8), host(2, K), host(2, N)
    raises_gpu(gq.gq_matvec, "q4_k", W, N, K, x, y)                  # all good but on the host
    with pytest.raises(ValueError, match="y holds"):
        gq.gq_matvec("q4_k", W, N, K, x, host(2, N - 1))             # short y
    with pytest.raises(ValueError, match="W holds"):
        gq.gq_matvec("q4_k", W[:-1], N, K, x, y)                     # short W
    with pytest.raises(ValueError, match="whole number"):
        gq.gq_matvec("q4_k", W, N, K, host(2 * K + 1), y)            # x not whole rows
    with pytest.raises(ValueError, match="contiguous"):
        gq.gq_matvec("q4_k", W, N, K, host(K, 2).t(), y)             # strided x
    with pytest.raises(TypeError, match="dtype"):
        gq.gq_matvec("q4_k", W, N, K, host(2, K, dtype=torch.float64), y)
    with pytest.raises(TypeError, match="dtype"):
        gq.gq_matvec("q4_k", W, N, K, x, host(2, N, dtype=bf16))     # y must be fp32
    with pytest.raises(TypeError, match="dtype"):
        gq.gq_matvec("q4_k", W.to(i32), N, K, x, y)                  # W must be bytes
    with pytest.raises(TypeError, match="torch.Tensor"):
        gq.gq_matvec("q4_k", W, N, K, [0.0] * K, y)


def test_matvec_glu_checks():
    N, K = 32, 2560
    W, x, h = host(N * RB["q4_k"], dtype=u8), host(1, K), host(1, N)
    raises_gpu(gq.gq_matvec_glu, "q4_k", W, W, N, K, x, "silu", h)
    with pytest.raises(ValueError, match="act"):
        gq.gq_matvec_glu("q4_k", W, W, N, K, x, "relu", h)
    with pytest.raises(ValueError, match="h holds"):
        gq.gq_matvec_glu("q4_k", W, W, N, K, x, "silu", host(1, N - 1))
    with pytest.raises(ValueError, match="W_up holds"):
        gq.gq_matvec_glu("q4_k", W, W[:100], N, K, x, "silu", h)


def test_matvec_id_checks():
    E, N, K, T, k = 8, 16, 2048, 3, 2
    ex = host(E * N * RB["q4_0"], dtype=u8)
    ids, ws = host(T, k, dtype=i32), host(4096, dtype=u8)
    x, y = host(T, K), host(T, k, N)
    raises_gpu(gq.gq_matvec_id, "q4_0", ex, E, N, K, ids, x, False, y, ws)
    with pytest.raises(ValueError, match="x must hold"):
        gq.gq_matvec_id("q4_0", ex, E, N, K, ids, host(T, k, K), False, y, ws)   # per-slot x, per-token call
    with pytest.raises(ValueError, match="x must hold"):
        gq.gq_matvec_id("q4_0", ex, E, N, K, ids, x, True, y, ws)                # per-token x, per-slot call
    with pytest.raises(ValueError, match="y holds"):
        gq.gq_matvec_id("q4_0", ex, E, N, K, ids, x, False, host(T, N), ws)      # unweighted needs T x k x N
    with pytest.raises(ValueError, match="route_w"):
        gq.gq_matvec_id("q4_0", ex, E, N, K, ids, x, False, host(T, N), ws, host(T))
    with pytest.raises(ValueError, match="experts holds"):
        gq.gq_matvec_id("q4_0", ex[:-1], E, N, K, ids, x, False, y, ws)
    with pytest.raises(TypeError, match="ids"):
        gq.gq_matvec_id("q4_0", ex, E, N, K, host(T, k, dtype=torch.int64), x, False, y, ws)
    with pytest.raises(ValueError, match="ids must be"):
        gq.gq_matvec_id("q4_0", ex, E, N, K, host(T * k, dtype=i32), x, False, y, ws)
    raises_gpu(gq.gq_matvec_id, "q4_0", ex, E, N, K, ids, x, False, host(T, N), ws, host(T, k))  # weighted: T x N


def test_matvec_id_glu_checks():
    E, N, K, T, k = 4, 16, 2048, 2, 2
    ex = host(E * N * RB["q4_0"], dtype=u8)
    ids, ws = host(T, k, dtype=i32), host(4096, dtype=u8)
    raises_gpu(gq.gq_matvec_id_glu, "q4_0", ex, ex, E, N, K, ids, host(T, K), "silu", host(T, k, N), ws)
    with pytest.raises(ValueError, match="h holds"):
        gq.gq_matvec_id_glu("q4_0", ex, ex, E, N, K, ids, host(T, K), "silu", host(T, N), ws)
    with pytest.raises(ValueError, match="x must hold"):
        gq.gq_matvec_id_glu("q4_0", ex, ex, E, N, K, ids, host(T + 1, K), "silu", host(T, k, N), ws)
    with pytest.raises(TypeError, match="ws"):
        gq.gq_matvec_id_glu("q4_0", ex, ex, E, N, K, ids, host(T, K), "silu", host(T, k, N), host(16, dtype=i32))


def test_matmul_checks():
    N, K, M = 64, 2560, 5
    W = host(N * RB["q4_k"], dtype=u8)
    X, Y = host(M, K, dtype=bf16), host(M, N)
    raises_gpu(gq.gq_matmul, "q4_k", W, N, K, X, Y)
    raises_gpu(gq.gq_matmul, "q4_k", W, N, K, host(M, K + 64, dtype=bf16)[:, :K], Y)  # row stride of its own
    with pytest.raises(ValueError, match="Y is"):
        gq.gq_matmul("q4_k", W, N, K, X, host(M - 1, N))              # too few rows of Y
    with pytest.raises(ValueError, match="Y is"):
        gq.gq_matmul("q4_k", W, N, K, X, host(M, N - 1))
    with pytest.raises(ValueError, match="fewer than K"):
        gq.gq_matmul("q4_k", W, N, K, host(M, K - 256, dtype=bf16), Y)
    with pytest.raises(ValueError, match="unit stride"):
        gq.gq_matmul("q4_k", W, N, K, host(K, M, dtype=bf16).t(), Y)
    with pytest.raises(ValueError, match="2-D"):
        gq.gq_matmul("q4_k", W, N, K, host(M * K, dtype=bf16), Y)
    with pytest.raises(TypeError, match="dtype"):
        gq.gq_matmul("q4_k", W, N, K, host(M, K), Y)                  # fp32 X


def test_dequant_and_route_checks():
    raises_gpu(gq.gq_dequant, "q4_k", host(2 * 144, dtype=u8), host(512))
    with pytest.raises(ValueError, match="sizes"):
        gq.gq_dequant("q4_k", host(2 * 144, dtype=u8), host(511))
    with pytest.raises(ValueError, match="contiguous"):
        gq.gq_dequant("q4_k", host(2 * 144, dtype=u8), host(1024)[::2])
    raises_gpu(gq.gq_route_topk, host(4, 16), 2, host(4, 2, dtype=i32), host(4, 2))
    with pytest.raises(ValueError, match="n_tokens"):
        gq.gq_route_topk(host(4, 16), 2, host(4, 3, dtype=i32), host(4, 2))
    with pytest.raises(TypeError, match="dtype"):
        gq.gq_route_topk(host(4, 16, dtype=bf16), 2, host(4, 2, dtype=i32), host(4, 2))
    with pytest.raises(TypeError, match="GPU tensor"):
        gq.gq_matvec_id_check(host(256, dtype=u8))
