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
# GQ_LIBGQ names another build of the library (bench.py --abba compares two
# builds in alternating fresh processes this way)
lib_path = os.environ.get("GQ_LIBGQ") or os.path.join(_PKG, "libgq.so")

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
if hasattr(_lib, "gq_matvec_id_noalloc"):  # (older builds, compared by bench.py --abba, lack the newer calls)
    _lib.gq_matvec_id_noalloc.argtypes = [ctypes.c_int, P, I32, I64, I64, P, I32, I32, P, ctypes.c_int, I32, P, P,
                                          P]
_lib.gq_matmul.argtypes = [ctypes.c_int, P, I64, I64, P, ctypes.c_int, I64, I64, P, I64, P]
_lib.gq_route_topk.argtypes = [P, I32, I32, I32, P, P, P]
if hasattr(_lib, "gq_route_topk_plan"):
    _lib.gq_route_topk_plan.argtypes = [P, I32, I32, I32, P, P, P, SZ, P]
if hasattr(_lib, "gq_route_matvec_id_glu"):
    _lib.gq_route_matvec_id_glu.argtypes = [ctypes.c_int, P, P, I32, I64, I64, P, I32, I32, P, P, P, ctypes.c_int,
                                            ctypes.c_int, P, ctypes.c_int, P, SZ, P]
_lib.gq_matvec_glu.argtypes = [ctypes.c_int, P, P, I64, I64, P, ctypes.c_int, I32, ctypes.c_int, P, ctypes.c_int, P]
_lib.gq_matvec_id_glu.argtypes = [ctypes.c_int, P, P, I32, I64, I64, P, I32, I32, P, ctypes.c_int, ctypes.c_int, P,
                                  ctypes.c_int, P, SZ, P]
ACTS = {"silu": 0, "gelu_tanh": 1}
for _f in ("gq_block_info", "gq_dequant", "gq_matvec", "gq_matvec_id_workspace", "gq_matvec_id", "gq_matvec_id_noalloc",
           "gq_matvec_id_check", "gq_matmul", "gq_route_topk", "gq_route_topk_plan", "gq_matvec_glu",
           "gq_matvec_id_glu", "gq_route_matvec_id_glu"):
    if hasattr(_lib, _f):
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


# weights per block and bytes per block of each type (gq_block_info)
_BLOCK = {1: (32, 18), 2: (256, 144), 3: (256, 210), 4: (256, 176)}


def _row_bytes(t, K: int) -> int:
    """Packed bytes of one row of K inputs (a lower bound when K is not a
    whole number of blocks, which the library rejects itself)."""
    qk, bb = _BLOCK.get(_type(t), (32, 0))
    return (K // qk) * bb if K > 0 else 0


# Checks made before any call into the library.  The C ABI sees only
# pointers, so a tensor on the wrong device, of the wrong element type or too
# small would become an out-of-bounds device access; these raise instead.
# Order: element type, then sizes and layout, then the device -- so that every
# mistake is reported the same way with or without a GPU.

def _need(cond: bool, msg: str, exc=ValueError) -> None:
    if not cond:
        raise exc(msg)


def _tensor(name: str, t, dtypes) -> torch.Tensor:
    _need(isinstance(t, torch.Tensor), "%s must be a torch.Tensor" % name, TypeError)
    _need(t.dtype in dtypes, "%s must have dtype %s, not %s" % (name, " or ".join(map(str, dtypes)), t.dtype),
          TypeError)
    return t


def _contig(name: str, t: torch.Tensor) -> None:
    _need(t.is_contiguous(), "%s must be contiguous" % name)


def _rows(name: str, t: torch.Tensor) -> None:
    """2-D with unit stride along a row (a row stride of its own is allowed)."""
    _need(t.dim() == 2, "%s must be 2-D" % name)
    _need(t.stride(1) == 1 or t.shape[1] <= 1, "%s must have unit stride along dim 1" % name)


def _on_gpu(**tensors) -> None:
    for name, t in tensors.items():
        if t is not None:
            _need(t.is_cuda, "%s must be a GPU tensor" % name, TypeError)


_F32, _ACT = (torch.float32,), (torch.float32, torch.bfloat16)
_U8, _I32 = (torch.uint8,), (torch.int32,)


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
    _tensor("blocks", blocks, _U8)
    _tensor("out", out, (torch.float32, torch.bfloat16, torch.float16))
    elems, nbytes = gq_block_info(t)
    n_blocks = blocks.numel() // nbytes
    _need(blocks.numel() == n_blocks * nbytes and out.numel() == n_blocks * elems, "blocks / out sizes do not match")
    _contig("blocks", blocks)
    _contig("out", out)
    _on_gpu(blocks=blocks, out=out)
    _check("gq_dequant", _lib.gq_dequant(_type(t), _ptr(blocks), n_blocks, _ptr(out), _DTYPES[out.dtype],
                                         _stream(stream)))
    return out


def _weights(name: str, W: torch.Tensor, t, rows: int, K: int) -> None:
    _tensor(name, W, _U8)
    _contig(name, W)
    _need(W.numel() >= rows * _row_bytes(t, K), "%s holds %d bytes, fewer than %d rows of K = %d"
          % (name, W.numel(), rows, K))


def _batch(x: torch.Tensor, K: int, N: int, out: torch.Tensor) -> int:
    if K:
        _need(x.numel() % K == 0 and x.numel() > 0, "x must hold a whole number (>= 1) of rows of K = %d" % K)
        return x.numel() // K
    return out.numel() // N if N else 1


def gq_matvec(t, W: torch.Tensor, N: int, K: int, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y[b][n] = sum_k w[n][k] x[b][k]; x is [batch][K] fp32/bf16, y [batch][N] fp32."""
    _tensor("x", x, _ACT)
    _tensor("y", y, _F32)
    _weights("W", W, t, N, K)
    _contig("x", x)
    _contig("y", y)
    batch = _batch(x, K, N, y)
    _need(y.numel() >= batch * N, "y holds %d elements, fewer than batch * N = %d" % (y.numel(), batch * N))
    _on_gpu(W=W, x=x, y=y)
    _check("gq_matvec", _lib.gq_matvec(_type(t), _ptr(W), N, K, _ptr(x), _DTYPES[x.dtype], batch, _ptr(y),
                                       _stream(stream)))
    return y


def gq_matvec_glu(t, W_gate: torch.Tensor, W_up: torch.Tensor, N: int, K: int, x: torch.Tensor, act: str,
                  h: torch.Tensor, stream=None) -> torch.Tensor:
    """h[b][n] = act(w_gate[n] . x[b]) * (w_up[n] . x[b]); x [batch][K] fp32/bf16, h [batch][N] fp32/bf16."""
    _tensor("x", x, _ACT)
    _tensor("h", h, _ACT)
    _need(act in ACTS, "act must be one of %s" % sorted(ACTS))
    _weights("W_gate", W_gate, t, N, K)
    _weights("W_up", W_up, t, N, K)
    _contig("x", x)
    _contig("h", h)
    batch = _batch(x, K, N, h)
    _need(h.numel() >= batch * N, "h holds %d elements, fewer than batch * N = %d" % (h.numel(), batch * N))
    _on_gpu(W_gate=W_gate, W_up=W_up, x=x, h=h)
    _check("gq_matvec_glu", _lib.gq_matvec_glu(_type(t), _ptr(W_gate), _ptr(W_up), N, K, _ptr(x), _DTYPES[x.dtype],
                                               batch, ACTS[act], _ptr(h), _DTYPES[h.dtype], _stream(stream)))
    return h


def gq_matvec_id_workspace(n_experts: int, n_tokens: int, top_k: int, N: int) -> int:
    b = SZ()
    _check("gq_matvec_id_workspace", _lib.gq_matvec_id_workspace(n_experts, n_tokens, top_k, N, ctypes.byref(b)))
    return b.value


def _ids(ids: torch.Tensor) -> tuple[int, int]:
    _tensor("ids", ids, _I32)
    _need(ids.dim() == 2, "ids must be [n_tokens][top_k]")
    _contig("ids", ids)
    return ids.shape[0], ids.shape[1]


def _workspace(ws: torch.Tensor) -> None:
    _tensor("ws", ws, _U8)
    _contig("ws", ws)


def gq_matvec_id(t, experts: torch.Tensor, n_experts: int, N: int, K: int, ids, x: torch.Tensor,
                 x_per_slot: bool, y: torch.Tensor, ws: torch.Tensor, route_w: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Routed product; x [n_tokens][K] (or [n_tokens][top_k][K] per slot), y
    [n_tokens][top_k][N] (or [n_tokens][N] weighted by route_w [n_tokens][top_k]).
    ids may be a (n_tokens, top_k) tuple instead of a tensor for a weighted
    product: the group table already in ws is used (ids NULL in the C call)."""
    reuse = isinstance(ids, tuple)
    n_tokens, top_k = ids if reuse else _ids(ids)
    _tensor("x", x, _ACT)
    _tensor("y", y, _F32)
    if route_w is not None:
        _tensor("route_w", route_w, _F32)
        _contig("route_w", route_w)
        _need(route_w.numel() >= n_tokens * top_k, "route_w must hold n_tokens * top_k elements")
    # nothing is read when there are no tokens or no rows (a no-op call)
    _weights("experts", experts, t, max(n_experts, 0) * N if n_tokens and N else 0, K)
    _workspace(ws)
    _contig("x", x)
    _contig("y", y)
    slots = n_tokens * (top_k if x_per_slot else 1)
    _need(x.numel() == slots * K, "x must hold %d x %d elements" % (slots, K))
    want_y = n_tokens * N * (1 if route_w is not None else top_k)
    _need(y.numel() >= want_y, "y holds %d elements, fewer than %d" % (y.numel(), want_y))
    _on_gpu(experts=experts, ids=None if reuse else ids, x=x, y=y, ws=ws, route_w=route_w)
    _check("gq_matvec_id", _lib.gq_matvec_id(_type(t), _ptr(experts), n_experts, N, K,
                                             None if reuse else _ptr(ids), n_tokens, top_k,
                                             _ptr(x), _DTYPES[x.dtype], 1 if x_per_slot else 0, _ptr(route_w),
                                             _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return y


def gq_matvec_id_noalloc(t, experts: torch.Tensor, n_experts: int, N: int, K: int, ids, x: torch.Tensor,
                         x_per_slot: bool, y: torch.Tensor, route_w: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """gq_matvec_id with the library's own per-GPU workspace (no allocation;
    ids may be a (n_tokens, top_k) tuple for a weighted product to reuse the
    previous call's group table)."""
    reuse = isinstance(ids, tuple)
    n_tokens, top_k = ids if reuse else _ids(ids)
    _tensor("x", x, _ACT)
    _tensor("y", y, _F32)
    if route_w is not None:
        _tensor("route_w", route_w, _F32)
        _contig("route_w", route_w)
        _need(route_w.numel() >= n_tokens * top_k, "route_w must hold n_tokens * top_k elements")
    _weights("experts", experts, t, max(n_experts, 0) * N if n_tokens and N else 0, K)
    _contig("x", x)
    _contig("y", y)
    slots = n_tokens * (top_k if x_per_slot else 1)
    _need(x.numel() == slots * K, "x must hold %d x %d elements" % (slots, K))
    want_y = n_tokens * N * (1 if route_w is not None else top_k)
    _need(y.numel() >= want_y, "y holds %d elements, fewer than %d" % (y.numel(), want_y))
    _on_gpu(experts=experts, ids=None if reuse else ids, x=x, y=y, route_w=route_w)
    _check("gq_matvec_id_noalloc", _lib.gq_matvec_id_noalloc(
        _type(t), _ptr(experts), n_experts, N, K, None if reuse else _ptr(ids), n_tokens, top_k, _ptr(x),
        _DTYPES[x.dtype], 1 if x_per_slot else 0, _ptr(route_w), _ptr(y), _stream(stream)))
    return y


def gq_matvec_id_glu(t, experts_gate: torch.Tensor, experts_up: torch.Tensor, n_experts: int, N: int, K: int,
                     ids: torch.Tensor, x: torch.Tensor, act: str, h: torch.Tensor, ws: torch.Tensor,
                     stream=None) -> torch.Tensor:
    """h[t][j][n] = act(gate_e[n] . x[t]) * (up_e[n] . x[t]) with e = ids[t][j]; h [n_tokens][top_k][N].
    ids may be a (n_tokens, top_k) tuple: the group table already in ws is used."""
    reuse = isinstance(ids, tuple)
    n_tokens, top_k = ids if reuse else _ids(ids)
    _tensor("x", x, _ACT)
    _tensor("h", h, _ACT)
    _need(act in ACTS, "act must be one of %s" % sorted(ACTS))
    rows = max(n_experts, 0) * N if n_tokens and N else 0  # a no-op call reads nothing
    _weights("experts_gate", experts_gate, t, rows, K)
    _weights("experts_up", experts_up, t, rows, K)
    _workspace(ws)
    _contig("x", x)
    _contig("h", h)
    _need(x.numel() == n_tokens * K, "x must hold n_tokens x K = %d x %d elements" % (n_tokens, K))
    _need(h.numel() >= n_tokens * top_k * N, "h holds %d elements, fewer than n_tokens * top_k * N" % h.numel())
    _on_gpu(experts_gate=experts_gate, experts_up=experts_up, ids=None if reuse else ids, x=x, h=h, ws=ws)
    _check("gq_matvec_id_glu", _lib.gq_matvec_id_glu(_type(t), _ptr(experts_gate), _ptr(experts_up), n_experts, N,
                                                     K, None if reuse else _ptr(ids), n_tokens, top_k, _ptr(x), _DTYPES[x.dtype],
                                                     ACTS[act], _ptr(h), _DTYPES[h.dtype], _ptr(ws),
                                                     ws.numel() * ws.element_size(), _stream(stream)))
    return h


def gq_matvec_id_check(ws: torch.Tensor, stream=None) -> int:
    _workspace(ws)
    _on_gpu(ws=ws)
    n = I32()
    _check("gq_matvec_id_check", _lib.gq_matvec_id_check(_ptr(ws), _stream(stream), ctypes.byref(n)))
    return n.value


def gq_matmul(t, W: torch.Tensor, N: int, K: int, X: torch.Tensor, Y: torch.Tensor, stream=None) -> torch.Tensor:
    """Y[m][n] = sum_k X[m][k] w[n][k]; X [M][ldx] bf16, Y [M][ldy] fp32 (2-D, unit
    stride along a row; the row strides are passed as ldx, ldy)."""
    _tensor("X", X, (torch.bfloat16,))
    _tensor("Y", Y, _F32)
    _weights("W", W, t, N, K)
    _rows("X", X)
    _rows("Y", Y)
    M = X.shape[0]
    _need(X.shape[1] >= K, "X rows hold %d elements, fewer than K = %d" % (X.shape[1], K))
    _need(Y.shape[0] >= M and Y.shape[1] >= N, "Y is %s, smaller than M x N = %d x %d" % (tuple(Y.shape), M, N))
    ldx = X.stride(0) if M > 1 else max(X.shape[1], K)
    ldy = Y.stride(0) if Y.shape[0] > 1 else max(Y.shape[1], N)
    _on_gpu(W=W, X=X, Y=Y)
    _check("gq_matmul", _lib.gq_matmul(_type(t), _ptr(W), N, K, _ptr(X), _DTYPES[X.dtype], M, ldx, _ptr(Y), ldy,
                                       _stream(stream)))
    return Y


def gq_route_topk(logits: torch.Tensor, top_k: int, ids: torch.Tensor, weights: torch.Tensor,
                  stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """ids / weights [n_tokens][top_k] (int32 / fp32) of the softmax + top-k
    routing of fp32 ``logits`` [n_tokens][n_experts]."""
    _tensor("logits", logits, _F32)
    _tensor("ids", ids, _I32)
    _tensor("weights", weights, _F32)
    _need(logits.dim() == 2, "logits must be [n_tokens][n_experts]")
    n_tokens, n_experts = logits.shape
    _need(ids.numel() == n_tokens * top_k and weights.numel() == n_tokens * top_k,
          "ids / weights must hold n_tokens * top_k elements")
    for name, v in (("logits", logits), ("ids", ids), ("weights", weights)):
        _contig(name, v)
    _on_gpu(logits=logits, ids=ids, weights=weights)
    _check("gq_route_topk", _lib.gq_route_topk(_ptr(logits), n_tokens, n_experts, top_k, _ptr(ids),
                                               _ptr(weights), _stream(stream)))
    return ids, weights


def gq_route_topk_plan(logits: torch.Tensor, top_k: int, ids: torch.Tensor, weights: torch.Tensor, ws: torch.Tensor,
                       stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """gq_route_topk plus the routed products' group table in ws (so that the
    products can take ids as a (n_tokens, top_k) tuple)."""
    _tensor("logits", logits, _F32)
    _tensor("ids", ids, _I32)
    _tensor("weights", weights, _F32)
    _need(logits.dim() == 2, "logits must be [n_tokens][n_experts]")
    n_tokens, n_experts = logits.shape
    _need(ids.numel() == n_tokens * top_k and weights.numel() == n_tokens * top_k,
          "ids / weights must hold n_tokens * top_k elements")
    for name, v in (("logits", logits), ("ids", ids), ("weights", weights)):
        _contig(name, v)
    _workspace(ws)
    _on_gpu(logits=logits, ids=ids, weights=weights, ws=ws)
    _check("gq_route_topk_plan", _lib.gq_route_topk_plan(_ptr(logits), n_tokens, n_experts, top_k, _ptr(ids),
                                                         _ptr(weights), _ptr(ws), ws.numel(), _stream(stream)))
    return ids, weights


def gq_route_matvec_id_glu(t, experts_gate: torch.Tensor, experts_up: torch.Tensor, n_experts: int, N: int, K: int,
                           logits: torch.Tensor, top_k: int, ids: torch.Tensor, weights: torch.Tensor, x: torch.Tensor,
                           act: str, h: torch.Tensor, ws: torch.Tensor, stream=None) -> torch.Tensor:
    """gq_route_topk_plan then gq_matvec_id_glu on the table it leaves (one
    launch where the sizes allow): ids, weights and h as those two calls write
    them; later products may take ids as a (n_tokens, top_k) tuple."""
    _tensor("logits", logits, _F32)
    _tensor("ids", ids, _I32)
    _tensor("weights", weights, _F32)
    _tensor("x", x, _ACT)
    _tensor("h", h, _ACT)
    _need(logits.dim() == 2 and logits.shape[1] == n_experts, "logits must be [n_tokens][n_experts]")
    n_tokens = logits.shape[0]
    _need(ids.numel() == n_tokens * top_k and weights.numel() == n_tokens * top_k,
          "ids / weights must hold n_tokens * top_k elements")
    _need(act in ACTS, "act must be one of %s" % sorted(ACTS))
    rows = max(n_experts, 0) * N if n_tokens and N else 0
    _weights("experts_gate", experts_gate, t, rows, K)
    _weights("experts_up", experts_up, t, rows, K)
    _workspace(ws)
    for name, v in (("logits", logits), ("ids", ids), ("weights", weights), ("x", x), ("h", h)):
        _contig(name, v)
    _need(x.numel() == n_tokens * K, "x must hold n_tokens x K = %d x %d elements" % (n_tokens, K))
    _need(h.numel() >= n_tokens * top_k * N, "h holds %d elements, fewer than n_tokens * top_k * N" % h.numel())
    _on_gpu(experts_gate=experts_gate, experts_up=experts_up, logits=logits, ids=ids, weights=weights, x=x, h=h, ws=ws)
    _check("gq_route_matvec_id_glu",
           _lib.gq_route_matvec_id_glu(_type(t), _ptr(experts_gate), _ptr(experts_up), n_experts, N, K, _ptr(logits),
                                       n_tokens, top_k, _ptr(ids), _ptr(weights), _ptr(x), _DTYPES[x.dtype], ACTS[act],
                                       _ptr(h), _DTYPES[h.dtype], _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)))
    return h


# raw handle for the tests that check the exported symbols
_cdll = _lib
