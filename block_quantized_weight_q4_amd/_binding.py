"""ctypes binding of libgq.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
data pointers and the current HIP stream to the C entry point of the same name
and raises :class:`GqError` on a non-zero status.  No computation happens here
and there is no fallback: if ``libgq.so`` is missing, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libgq.so")

if not os.path.exists(lib_path):
    raise ImportError(
        "libgq.so is not built (expected at %s); run `python -m block_quantized_weight_q4_amd.build`" % lib_path)

_lib = ctypes.CDLL(lib_path)

TYPES = {"q4_0": 1, "q4_k": 2, "q6_k": 3, "q5_k": 4}
_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
_STATUS = {}

P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_lib.gq_abi_version.restype = ctypes.c_int
_lib.gq_status_str.argtypes = [ctypes.c_int]
_lib.gq_status_str.restype = ctypes.c_char_p
_lib.gq_block_info.argtypes = [ctypes.c_int, ctypes.POINTER(I32), ctypes.POINTER(I32)]
_lib.gq_dequant.argtypes = [ctypes.c_int, P, I64, P, ctypes.c_int, P]
_lib.gq_matvec.argtypes = [ctypes.c_int, P, I64, I64, P, ctypes.c_int, I32, P, P]
_lib.gq_matvec_id_workspace.argtypes = [I32, I32, I32, I64, ctypes.POINTER(SZ)]
_lib.gq_matvec_id.argtypes = [ctypes.c_int, P, I32, I64, I64, P, I32, I32, P, ctypes.c_int, I32, P, P, P, SZ, P]
_lib.gq_matvec_id_check.argtypes = [P, P, ctypes.POINTER(I32)]
_lib.gq_matmul.argtypes = [ctypes.c_int, P, I64, I64, P, ctypes.c_int, I64, I64, P, I64, P]
_lib.gq_route_topk.argtypes = [P, I32, I32, I32, P, P, P]
_lib.gq_matvec_glu.argtypes = [ctypes.c_int, P, P, I64, I64, P, ctypes.c_int, I32, ctypes.c_int, P, ctypes.c_int, P]
_lib.gq_matvec_id_glu.argtypes = [ctypes.c_int, P, P, I32, I64, I64, P, I32, I32, P, ctypes.c_int, ctypes.c_int, P,
                                  ctypes.c_int, P, SZ, P]
ACTS = {"silu": 0, "gelu_tanh": 1}
for _f in ("gq_block_info", "gq_dequant", "gq_matvec", "gq_matvec_id_workspace", "gq_matvec_id",
           "gq_matvec_id_check", "gq_matmul", "gq_route_topk", "gq_matvec_glu", "gq_matvec_id_glu"):
    getattr(_lib, _f).restype = ctypes.c_int


class GqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.gq_status_str(status).decode()
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise GqError(fn, status)


def _type(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def gq_abi_version() -> int:
    return int(_lib.gq_abi_version())


def gq_block_info(t) -> tuple[int, int]:
    e, b = I32(), I32()
    _check("gq_block_info", _lib.gq_block_info(_type(t), ctypes.byref(e), ctypes.byref(b)))
    return e.value, b.value


def gq_dequant(t, blocks: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """out[:] = weights of the packed ``blocks`` (uint8, whole blocks)."""
    elems, nbytes = gq_block_info(t)
    n_blocks = blocks.numel() // nbytes
    if blocks.numel() != n_blocks * nbytes or out.numel() != n_blocks * elems:
        raise ValueError("blocks / out sizes do not match")
    _check("gq_dequant", _lib.gq_dequant(_type(t), _ptr(blocks), n_blocks, _ptr(out), _DTYPES[out.dtype],
                                         _stream(stream)))
    return out


def gq_matvec(t, W: torch.Tensor, N: int, K: int, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y[b][n] = sum_k w[n][k] x[b][k]; x is [batch][K] fp32/bf16, y [batch][N] fp32."""
    batch = x.numel() // K if K else (y.numel() // N if N else 1)
    _check("gq_matvec", _lib.gq_matvec(_type(t), _ptr(W), N, K, _ptr(x), _DTYPES[x.dtype], batch, _ptr(y),
                                       _stream(stream)))
    return y


def gq_matvec_glu(t, W_gate: torch.Tensor, W_up: torch.Tensor, N: int, K: int, x: torch.Tensor, act: str,
                  h: torch.Tensor, stream=None) -> torch.Tensor:
    """h[b][n] = act(w_gate[n] . x[b]) * (w_up[n] . x[b]); x [batch][K] fp32/bf16, h [batch][N] fp32/bf16."""
    batch = x.numel() // K if K else (h.numel() // N if N else 1)
    _check("gq_matvec_glu", _lib.gq_matvec_glu(_type(t), _ptr(W_gate), _ptr(W_up), N, K, _ptr(x), _DTYPES[x.dtype],
                                               batch, ACTS[act], _ptr(h), _DTYPES[h.dtype], _stream(stream)))
    return h


def gq_matvec_id_workspace(n_experts: int, n_tokens: int, top_k: int, N: int) -> int:
    b = SZ()
    _check("gq_matvec_id_workspace", _lib.gq_matvec_id_workspace(n_experts, n_tokens, top_k, N, ctypes.byref(b)))
    return b.value


def gq_matvec_id(t, experts: torch.Tensor, n_experts: int, N: int, K: int, ids: torch.Tensor, x: torch.Tensor,
                 x_per_slot: bool, y: torch.Tensor, ws: torch.Tensor, route_w: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    n_tokens, top_k = ids.shape
    _check("gq_matvec_id", _lib.gq_matvec_id(_type(t), _ptr(experts), n_experts, N, K, _ptr(ids), n_tokens, top_k,
                                             _ptr(x), _DTYPES[x.dtype], 1 if x_per_slot else 0, _ptr(route_w),
                                             _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return y


def gq_matvec_id_glu(t, experts_gate: torch.Tensor, experts_up: torch.Tensor, n_experts: int, N: int, K: int,
                     ids: torch.Tensor, x: torch.Tensor, act: str, h: torch.Tensor, ws: torch.Tensor,
                     stream=None) -> torch.Tensor:
    """h[t][j][n] = act(gate_e[n] . x[t]) * (up_e[n] . x[t]) with e = ids[t][j]; h [n_tokens][top_k][N]."""
    n_tokens, top_k = ids.shape
    _check("gq_matvec_id_glu", _lib.gq_matvec_id_glu(_type(t), _ptr(experts_gate), _ptr(experts_up), n_experts, N,
                                                     K, _ptr(ids), n_tokens, top_k, _ptr(x), _DTYPES[x.dtype],
                                                     ACTS[act], _ptr(h), _DTYPES[h.dtype], _ptr(ws),
                                                     ws.numel() * ws.element_size(), _stream(stream)))
    return h


def gq_matvec_id_check(ws: torch.Tensor, stream=None) -> int:
    n = I32()
    _check("gq_matvec_id_check", _lib.gq_matvec_id_check(_ptr(ws), _stream(stream), ctypes.byref(n)))
    return n.value


def gq_matmul(t, W: torch.Tensor, N: int, K: int, X: torch.Tensor, Y: torch.Tensor, stream=None) -> torch.Tensor:
    """Y[m][n] = sum_k X[m][k] w[n][k]; X [M][ldx] bf16, Y [M][ldy] fp32."""
    M = X.shape[0]
    ldx = X.stride(0) if X.dim() == 2 else K
    ldy = Y.stride(0) if Y.dim() == 2 else N
    _check("gq_matmul", _lib.gq_matmul(_type(t), _ptr(W), N, K, _ptr(X), _DTYPES[X.dtype], M, ldx, _ptr(Y), ldy,
                                       _stream(stream)))
    return Y


def gq_route_topk(logits: torch.Tensor, top_k: int, ids: torch.Tensor, weights: torch.Tensor,
                  stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """ids / weights [n_tokens][top_k] (int32 / fp32) of the softmax + top-k
    routing of fp32 ``logits`` [n_tokens][n_experts]."""
    n_tokens, n_experts = logits.shape
    if logits.dtype != torch.float32 or ids.dtype != torch.int32 or weights.dtype != torch.float32:
        raise TypeError("logits and weights must be float32, ids int32")
    if ids.numel() != n_tokens * top_k or weights.numel() != n_tokens * top_k:
        raise ValueError("ids / weights must hold n_tokens * top_k elements")
    _check("gq_route_topk", _lib.gq_route_topk(_ptr(logits), n_tokens, n_experts, top_k, _ptr(ids),
                                               _ptr(weights), _stream(stream)))
    return ids, weights


# raw handle for the tests that check the exported symbols
_cdll = _lib
