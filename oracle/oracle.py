"""CPU oracle: numpy front end for ``gq_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It never imports the
GPU package and the GPU package never imports it.

Every function takes and returns numpy arrays.  Packed weights are ``uint8``
arrays of whole blocks; activations are fp32 (bf16 inputs are expanded exactly
to fp32 by the caller); results are fp64 together with ``sum |w*x|`` per
element, from which the per-element tolerance ``1e-3 * sum|w*x|`` is formed by
the caller.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q4_0, Q4_K, Q6_K, Q5_K = 1, 2, 3, 4
TYPES = {"q4_0": Q4_0, "q4_k": Q4_K, "q6_k": Q6_K, "q5_k": Q5_K}

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, no vectorisation flags)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _setup(cdll):
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    cdll.oracle_block_info.argtypes = [ctypes.c_int, ctypes.POINTER(I32), ctypes.POINTER(I32)]
    cdll.oracle_dequant.argtypes = [ctypes.c_int, P, I64, P]
    cdll.oracle_matvec_rows.argtypes = [ctypes.c_int, P, I64, I64, P, I32, I64, I64, P, P]
    cdll.oracle_matvec_id.argtypes = [ctypes.c_int, P, I32, I64, I64, P, I32, I32, P, I32, P, P, P]
    cdll.oracle_matmul_rows.argtypes = [ctypes.c_int, P, I64, I64, P, I64, P, I64, P, P]
    cdll.oracle_matmul_cols.argtypes = [ctypes.c_int, P, I64, I64, P, I64, I64, P, I64, P, P]
    cdll.oracle_matmul_checksum.argtypes = [ctypes.c_int, P, I64, I64, P, I64, I64, P, P,
                                            ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_double)]
    cdll.oracle_quantize.argtypes = [ctypes.c_int, P, I64, P]
    cdll.oracle_route_topk.argtypes = [P, I32, I32, I32, P, P]
    cdll.oracle_glu.argtypes = [P, P, I64, ctypes.c_int, P]
    cdll.oracle_half_to_float.argtypes = [ctypes.c_uint16]
    cdll.oracle_half_to_float.restype = ctypes.c_float
    cdll.oracle_float_to_half.argtypes = [ctypes.c_float]
    cdll.oracle_float_to_half.restype = ctypes.c_uint16
    return cdll


def lib():
    global _lib
    if _lib is None:
        _lib = _setup(ctypes.CDLL(build()))
    return _lib


class using:
    """Context manager that routes this module's functions through another
    build of the oracle (the tests use it to check that planted mistakes are
    caught by the pins)."""

    def __init__(self, so_path: str):
        self.cdll = _setup(ctypes.CDLL(so_path))

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = self.cdll
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def build_variant(src_text: str, out_path: str) -> str:
    """Compile a (modified) copy of the oracle source with the same flags."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *CFLAGS, c_path, "-o", out_path, "-lm"])
    return out_path


def source() -> str:
    with open(_SRC) as f:
        return f.read()


def _t(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def block_info(t) -> tuple[int, int]:
    e, b = ctypes.c_int32(), ctypes.c_int32()
    if lib().oracle_block_info(_t(t), ctypes.byref(e), ctypes.byref(b)):
        raise ValueError("unknown type %r" % (t,))
    return e.value, b.value


def dequant(t, blocks: np.ndarray) -> np.ndarray:
    """fp32 weights of every block, in order (bit-exact target)."""
    elems, nbytes = block_info(t)
    blocks = _c(blocks, np.uint8).reshape(-1)
    if blocks.size % nbytes:
        raise ValueError("byte count is not a whole number of blocks")
    nb = blocks.size // nbytes
    out = np.empty(nb * elems, np.float32)
    if lib().oracle_dequant(_t(t), _p(blocks), nb, _p(out)):
        raise RuntimeError("oracle_dequant failed")
    return out


def matvec(t, W: np.ndarray, N: int, K: int, x: np.ndarray, rows=None):
    """y[b][n] and sum|w*x|[b][n] in fp64.  ``rows=(r0, r1)`` limits the rows
    computed (others are left NaN)."""
    x = _c(x, np.float32).reshape(-1, K)
    W = _c(W, np.uint8).reshape(-1)
    batch = x.shape[0]
    r0, r1 = (0, N) if rows is None else rows
    y = np.full((batch, N), np.nan)
    a = np.full((batch, N), np.nan)
    if lib().oracle_matvec_rows(_t(t), _p(W), N, K, _p(x), batch, r0, r1, _p(y), _p(a)):
        raise RuntimeError("oracle_matvec_rows failed")
    return y, a


def matvec_id(t, experts: np.ndarray, n_experts: int, N: int, K: int, ids: np.ndarray,
              x: np.ndarray, x_per_slot: bool, route_w=None):
    ids = _c(ids, np.int32)
    n_tokens, top_k = ids.shape
    x = _c(x, np.float32)
    experts = _c(experts, np.uint8).reshape(-1)
    if route_w is None:
        shape = (n_tokens, top_k, N)
        rw = None
    else:
        shape = (n_tokens, N)
        rw = _c(route_w, np.float32)
    y = np.empty(shape)
    a = np.empty(shape)
    rc = lib().oracle_matvec_id(_t(t), _p(experts), n_experts, N, K, _p(ids), n_tokens, top_k,
                                _p(x), 1 if x_per_slot else 0, None if rw is None else _p(rw),
                                _p(y), _p(a))
    if rc:
        raise RuntimeError("oracle_matvec_id failed")
    return y, a


def route_topk(logits: np.ndarray, top_k: int):
    """(ids int32 [T][k], weights fp64 [T][k]) of the softmax + top-k routing."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k))
    if lib().oracle_route_topk(_p(logits), T, E, top_k, _p(ids), _p(w)):
        raise RuntimeError("oracle_route_topk failed")
    return ids, w


def glu(g: np.ndarray, u: np.ndarray, act: str) -> np.ndarray:
    """h = act(g) * u elementwise in fp64; act "silu" or "gelu_tanh"."""
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    assert g.shape == u.shape
    h = np.empty(g.shape)
    if lib().oracle_glu(_p(g), _p(u), g.size, {"silu": 0, "gelu_tanh": 1}[act], _p(h)):
        raise RuntimeError("oracle_glu failed")
    return h


def matmul_rows(t, W: np.ndarray, N: int, K: int, X: np.ndarray, rows):
    X = _c(X, np.float32)
    rows = _c(rows, np.int64)
    y = np.empty((rows.size, N))
    a = np.empty((rows.size, N))
    if lib().oracle_matmul_rows(_t(t), _p(_c(W, np.uint8)), N, K, _p(X), X.shape[1], _p(rows),
                                rows.size, _p(y), _p(a)):
        raise RuntimeError("oracle_matmul_rows failed")
    return y, a


def matmul_cols(t, W: np.ndarray, N: int, K: int, X: np.ndarray, cols):
    X = _c(X, np.float32)
    cols = _c(cols, np.int64)
    M = X.shape[0]
    y = np.empty((M, cols.size))
    a = np.empty((M, cols.size))
    if lib().oracle_matmul_cols(_t(t), _p(_c(W, np.uint8)), N, K, _p(X), M, X.shape[1], _p(cols),
                                cols.size, _p(y), _p(a)):
        raise RuntimeError("oracle_matmul_cols failed")
    return y, a


def matmul_checksum(t, W: np.ndarray, N: int, K: int, X: np.ndarray, u: np.ndarray, v: np.ndarray):
    """(u^T Y v, tolerance term) without forming Y."""
    X = _c(X, np.float32)
    u = _c(u, np.float64)
    v = _c(v, np.float64)
    c, tt = ctypes.c_double(), ctypes.c_double()
    if lib().oracle_matmul_checksum(_t(t), _p(_c(W, np.uint8)), N, K, _p(X), X.shape[0], X.shape[1],
                                    _p(u), _p(v), ctypes.byref(c), ctypes.byref(tt)):
        raise RuntimeError("oracle_matmul_checksum failed")
    return c.value, tt.value


def quantize(t, x: np.ndarray) -> np.ndarray:
    elems, nbytes = block_info(t)
    x = _c(x, np.float32).reshape(-1)
    if x.size % elems:
        raise ValueError("length is not a whole number of blocks")
    nb = x.size // elems
    out = np.zeros(nb * nbytes, np.uint8)
    if lib().oracle_quantize(_t(t), _p(x), nb, _p(out)):
        raise RuntimeError("oracle_quantize failed")
    return out


def half_to_float(h: int) -> float:
    return float(lib().oracle_half_to_float(int(h) & 0xFFFF))


def float_to_half(f: float) -> int:
    return int(lib().oracle_float_to_half(float(f)))
