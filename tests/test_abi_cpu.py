"""The C ABI without a GPU: the library loads, exports every entry point that
include/gq.h declares, and rejects invalid arguments on the host -- before any
HIP call -- with the documented status codes.  No call here launches work:
every call either fails validation or is a documented no-op."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

GQ_OK, GQ_ERR_TYPE, GQ_ERR_DTYPE, GQ_ERR_SHAPE, GQ_ERR_NULL, GQ_ERR_ALIGN, GQ_ERR_UNSUPPORTED, \
    GQ_ERR_WORKSPACE, GQ_ERR_LAUNCH = range(9)

A = 0x10000  # fake, 16-byte aligned "device" address: never dereferenced
MIS = 0x10008  # 8-byte aligned only


@pytest.fixture(scope="module")
def lib(gq_lib_path):
    L = ctypes.CDLL(gq_lib_path)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.gq_status_str.restype = ctypes.c_char_p
    L.gq_dequant.argtypes = [ctypes.c_int, P, I64, P, ctypes.c_int, P]
    L.gq_matvec.argtypes = [ctypes.c_int, P, I64, I64, P, ctypes.c_int, I32, P, P]
    L.gq_matvec_id_workspace.argtypes = [I32, I32, I32, I64, ctypes.POINTER(SZ)]
    L.gq_matvec_id.argtypes = [ctypes.c_int, P, I32, I64, I64, P, I32, I32, P, ctypes.c_int, I32, P, P, P, SZ, P]
    L.gq_matvec_id_check.argtypes = [P, P, ctypes.POINTER(I32)]
    L.gq_matvec_id_noalloc.argtypes = [ctypes.c_int, P, I32, I64, I64, P, I32, I32, P, ctypes.c_int, I32, P, P, P]
    L.gq_matmul.argtypes = [ctypes.c_int, P, I64, I64, P, ctypes.c_int, I64, I64, P, I64, P]
    L.gq_block_info.argtypes = [ctypes.c_int, ctypes.POINTER(I32), ctypes.POINTER(I32)]
    L.gq_route_topk.argtypes = [P, I32, I32, I32, P, P, P]
    L.gq_route_topk_plan.argtypes = [P, I32, I32, I32, P, P, P, SZ, P]
    L.gq_matvec_glu.argtypes = [ctypes.c_int, P, P, I64, I64, P, ctypes.c_int, I32, ctypes.c_int, P, ctypes.c_int, P]
    L.gq_matvec_id_glu.argtypes = [ctypes.c_int, P, P, I32, I64, I64, P, I32, I32, P, ctypes.c_int, ctypes.c_int, P,
                                   ctypes.c_int, P, SZ, P]
    L.gq_route_matvec_id_glu.argtypes = [ctypes.c_int, P, P, I32, I64, I64, P, I32, I32, P, P, P, ctypes.c_int,
                                         ctypes.c_int, P, ctypes.c_int, P, SZ, P]
    return L


def declared_functions() -> list[str]:
    text = open(os.path.join(ROOT, "include", "gq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gq_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 15, names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.gq_abi_version() == 1
    for s in range(9):
        assert lib.gq_status_str(s)
    assert lib.gq_status_str(GQ_OK) == b"ok"


def test_block_info(lib):
    e, b = ctypes.c_int32(), ctypes.c_int32()
    for t, want in ((1, (32, 18)), (2, (256, 144)), (3, (256, 210)), (4, (256, 176))):
        assert lib.gq_block_info(t, ctypes.byref(e), ctypes.byref(b)) == GQ_OK
        assert (e.value, b.value) == want
    assert lib.gq_block_info(5, ctypes.byref(e), ctypes.byref(b)) == GQ_ERR_TYPE
    assert lib.gq_block_info(0, ctypes.byref(e), ctypes.byref(b)) == GQ_ERR_TYPE
    assert lib.gq_block_info(2, None, ctypes.byref(b)) == GQ_ERR_NULL


def test_dequant_validation(lib):
    assert lib.gq_dequant(7, A, 4, A, 0, None) == GQ_ERR_TYPE
    assert lib.gq_dequant(2, A, 4, A, 5, None) == GQ_ERR_DTYPE
    assert lib.gq_dequant(2, A, -1, A, 0, None) == GQ_ERR_SHAPE
    assert lib.gq_dequant(2, None, 4, A, 0, None) == GQ_ERR_NULL
    assert lib.gq_dequant(2, A, 4, None, 0, None) == GQ_ERR_NULL
    assert lib.gq_dequant(2, MIS, 4, A, 0, None) == GQ_ERR_ALIGN
    assert lib.gq_dequant(2, A, 4, MIS, 0, None) == GQ_ERR_ALIGN
    assert lib.gq_dequant(2, None, 0, None, 0, None) == GQ_OK  # empty: no-op


def test_matvec_validation(lib):
    mv = lib.gq_matvec
    assert mv(0, A, 8, 256, A, 0, 1, A, None) == GQ_ERR_TYPE
    assert mv(2, A, 8, 256, A, 2, 1, A, None) == GQ_ERR_DTYPE  # fp16 activations not offered
    assert mv(2, A, 8, 100, A, 0, 1, A, None) == GQ_ERR_SHAPE  # K not whole blocks
    assert mv(1, A, 8, 48, A, 0, 1, A, None) == GQ_ERR_SHAPE
    assert mv(2, A, -1, 256, A, 0, 1, A, None) == GQ_ERR_SHAPE
    assert mv(2, A, 8, -256, A, 0, 1, A, None) == GQ_ERR_SHAPE
    assert mv(2, A, 8, 256, A, 0, 0, A, None) == GQ_ERR_SHAPE
    assert mv(2, A, 8, 256, A, 0, 17, A, None) == GQ_ERR_UNSUPPORTED
    assert mv(2, None, 8, 256, A, 0, 1, A, None) == GQ_ERR_NULL
    assert mv(2, A, 8, 256, None, 0, 1, A, None) == GQ_ERR_NULL
    assert mv(2, A, 8, 256, A, 0, 1, None, None) == GQ_ERR_NULL
    assert mv(2, MIS, 8, 256, A, 0, 1, A, None) == GQ_ERR_ALIGN
    assert mv(2, A, 8, 256, MIS, 0, 1, A, None) == GQ_ERR_ALIGN
    assert mv(2, A, 8, 256, A, 0, 1, MIS, None) == GQ_ERR_ALIGN
    assert mv(2, A, 0, 256, A, 0, 1, A, None) == GQ_OK  # N == 0: no-op
    assert mv(3, A, 1 << 41, 256, A, 0, 1, A, None) == GQ_ERR_SHAPE  # size guard
    assert mv(2, A, 8, (1 << 22) + 256, A, 0, 1, A, None) == GQ_ERR_SHAPE  # longest decode row


def test_matvec_id_validation(lib):
    sz = ctypes.c_size_t()
    # the workspace is sized for exactly the call below (N = 704)
    assert lib.gq_matvec_id_workspace(128, 8, 8, 704, ctypes.byref(sz)) == GQ_OK
    need = sz.value
    assert need > 0
    assert lib.gq_matvec_id_workspace(4, 8, 8, 64, ctypes.byref(sz)) == GQ_ERR_SHAPE  # top_k > experts
    assert lib.gq_matvec_id_workspace(128, 129, 8, 64, ctypes.byref(sz)) == GQ_ERR_SHAPE  # > 1024 slots
    assert lib.gq_matvec_id_workspace(128, 8, 8, 64, None) == GQ_ERR_NULL
    f = lib.gq_matvec_id
    args = [1, A, 128, 704, 2816, A, 8, 8, A, 0, 0, None, A, A, need, None]

    def call(**kw):
        a = list(args)
        names = ["t", "ex", "E", "N", "K", "ids", "T", "k", "x", "xd", "per", "rw", "y", "ws", "wsb", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(t=5) == GQ_ERR_TYPE
    assert call(xd=2) == GQ_ERR_DTYPE
    assert call(K=2817) == GQ_ERR_SHAPE
    assert call(K=(1 << 22) + 32) == GQ_ERR_SHAPE
    assert call(k=129) == GQ_ERR_SHAPE
    assert call(E=0) == GQ_ERR_SHAPE
    assert call(per=2) == GQ_ERR_SHAPE
    assert call(T=129) == GQ_ERR_SHAPE  # 129 * 8 > 1024 slots
    # ids may be NULL (the table in ws is used): accepted up to the workspace check
    assert call(ids=None, wsb=0) == GQ_ERR_WORKSPACE
    assert call(ids=None, rw=A, wsb=0) == GQ_ERR_WORKSPACE
    assert call(ids=MIS) == GQ_ERR_ALIGN
    assert call(ws=None) == GQ_ERR_NULL
    assert call(y=MIS) == GQ_ERR_ALIGN
    assert call(rw=MIS) == GQ_ERR_ALIGN
    assert call(wsb=need - 1) == GQ_ERR_WORKSPACE
    assert call(wsb=0) == GQ_ERR_WORKSPACE
    assert call(T=0) == GQ_OK  # no tokens: no-op
    n = ctypes.c_int32()
    assert lib.gq_matvec_id_check(None, None, ctypes.byref(n)) == GQ_ERR_NULL
    assert lib.gq_matvec_id_check(MIS, None, ctypes.byref(n)) == GQ_ERR_ALIGN


def test_matmul_validation(lib):
    mm = lib.gq_matmul
    assert mm(9, A, 64, 256, A, 1, 16, 256, A, 64, None) == GQ_ERR_TYPE
    assert mm(2, A, 64, 256, A, 2, 16, 256, A, 64, None) == GQ_ERR_DTYPE
    assert mm(2, A, 64, 300, A, 1, 16, 300, A, 64, None) == GQ_ERR_SHAPE
    assert mm(2, A, 64, 256, A, 1, 16, 255, A, 64, None) == GQ_ERR_SHAPE  # ldx < K
    assert mm(2, A, 64, 256, A, 1, 16, 256, A, 63, None) == GQ_ERR_SHAPE  # ldy < N
    assert mm(2, A, 64, 256, A, 1, -1, 256, A, 64, None) == GQ_ERR_SHAPE
    assert mm(1, A, 64, 48, A, 1, 16, 48, A, 64, None) == GQ_ERR_SHAPE  # Q4_0: whole 32-blocks
    assert mm(2, A, 64, 256, A, 0, 16, 256, A, 64, None) == GQ_ERR_UNSUPPORTED
    assert mm(2, None, 64, 256, A, 1, 16, 256, A, 64, None) == GQ_ERR_NULL
    assert mm(2, A, 64, 256, A, 1, 16, 256, MIS, 64, None) == GQ_ERR_ALIGN
    assert mm(2, A, 64, 256, A, 1, 16, 260, A, 64, None) == GQ_ERR_ALIGN  # row stride breaks alignment
    assert mm(2, A, 64, 256, A, 1, 0, 256, A, 64, None) == GQ_OK  # M == 0: no-op
    assert mm(2, A, 0, 256, A, 1, 16, 256, A, 64, None) == GQ_OK  # N == 0: no-op


def test_binding_refuses_without_library(tmp_path, monkeypatch):
    """The Python binding has no fallback: with the library gone it raises."""
    import importlib.util
    import shutil
    pkg = os.path.join(ROOT, "block_quantized_weight_q4_amd")
    fake = tmp_path / "block_quantized_weight_q4_amd"
    fake.mkdir()
    for f in ("__init__.py", "_binding.py"):
        shutil.copy(os.path.join(pkg, f), fake / f)
    spec = importlib.util.spec_from_file_location("fakepkg._binding", fake / "_binding.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="libgq.so is not built"):
        spec.loader.exec_module(mod)


def test_route_topk_validation(lib):
    r = lib.gq_route_topk
    assert r(A, -1, 128, 8, A, A, None) == GQ_ERR_SHAPE
    assert r(A, 8, 0, 1, A, A, None) == GQ_ERR_SHAPE
    assert r(A, 8, 128, 0, A, A, None) == GQ_ERR_SHAPE
    assert r(A, 8, 4, 5, A, A, None) == GQ_ERR_SHAPE  # top_k > n_experts
    assert r(A, 8, 4097, 8, A, A, None) == GQ_ERR_UNSUPPORTED
    assert r(A, 8, 128, 65, A, A, None) == GQ_ERR_UNSUPPORTED
    assert r(None, 8, 128, 8, A, A, None) == GQ_ERR_NULL
    assert r(A, 8, 128, 8, None, A, None) == GQ_ERR_NULL
    assert r(A, 8, 128, 8, A, None, None) == GQ_ERR_NULL
    assert r(MIS, 8, 128, 8, A, A, None) == GQ_ERR_ALIGN
    assert r(A, 8, 128, 8, MIS, A, None) == GQ_ERR_ALIGN
    assert r(A, 8, 128, 8, A, MIS, None) == GQ_ERR_ALIGN
    assert r(None, 0, 128, 8, None, None, None) == GQ_OK  # no tokens: no-op


def test_matvec_glu_validation(lib):
    f = lib.gq_matvec_glu
    assert f(9, A, A, 8, 256, A, 0, 1, 0, A, 0, None) == GQ_ERR_TYPE
    assert f(2, A, A, 8, 256, A, 2, 1, 0, A, 0, None) == GQ_ERR_DTYPE  # fp16 activations
    assert f(2, A, A, 8, 256, A, 0, 1, 0, A, 2, None) == GQ_ERR_DTYPE  # fp16 output
    assert f(2, A, A, 8, 100, A, 0, 1, 0, A, 0, None) == GQ_ERR_SHAPE
    assert f(2, A, A, 8, 256, A, 0, 0, 0, A, 0, None) == GQ_ERR_SHAPE
    assert f(2, A, A, 8, (1 << 22) + 256, A, 0, 1, 0, A, 0, None) == GQ_ERR_SHAPE
    assert f(2, A, A, 8, 256, A, 0, 9, 0, A, 0, None) == GQ_ERR_UNSUPPORTED
    assert f(2, A, A, 8, 256, A, 0, 1, 2, A, 0, None) == GQ_ERR_UNSUPPORTED  # unknown activation
    assert f(2, None, A, 8, 256, A, 0, 1, 0, A, 0, None) == GQ_ERR_NULL
    assert f(2, A, None, 8, 256, A, 0, 1, 0, A, 0, None) == GQ_ERR_NULL
    assert f(2, A, A, 8, 256, A, 0, 1, 0, None, 0, None) == GQ_ERR_NULL
    assert f(2, A, MIS, 8, 256, A, 0, 1, 0, A, 0, None) == GQ_ERR_ALIGN
    assert f(2, A, A, 8, 256, A, 0, 1, 0, MIS, 1, None) == GQ_ERR_ALIGN
    assert f(2, A, A, 0, 256, A, 0, 1, 0, A, 0, None) == GQ_OK  # N == 0: no-op


def test_matvec_id_glu_validation(lib):
    f = lib.gq_matvec_id_glu
    # (type, gate, up, n_experts, N, K, ids, n_tokens, top_k, x, x_dtype, act, h, h_dtype, ws, ws_bytes, stream)
    ok = [2, A, A, 128, 704, 2816, A, 8, 8, A, 0, 0, A, 0, A, 1 << 30, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a0=9) == GQ_ERR_TYPE
    assert call(a10=2) == GQ_ERR_DTYPE  # fp16 activations
    assert call(a13=2) == GQ_ERR_DTYPE  # fp16 output
    assert call(a5=100) == GQ_ERR_SHAPE  # K not whole blocks
    assert call(a3=0) == GQ_ERR_SHAPE
    assert call(a8=0) == GQ_ERR_SHAPE
    assert call(a8=129) == GQ_ERR_SHAPE  # top_k > n_experts
    assert call(a7=129) == GQ_ERR_SHAPE  # 129 * 8 slots > 1024
    assert call(a5=(1 << 22) + 256) == GQ_ERR_SHAPE
    assert call(a11=2) == GQ_ERR_UNSUPPORTED  # unknown activation
    for i in (1, 2, 9, 12, 14):
        assert call(**{"a%d" % i: None}) == GQ_ERR_NULL, i
    assert call(a6=None, a15=0) == GQ_ERR_WORKSPACE  # NULL ids (the table in ws is used) pass validation
    for i in (1, 2, 6, 9, 12, 14):
        assert call(**{"a%d" % i: MIS}) == GQ_ERR_ALIGN, i
    need = ctypes.c_size_t()
    assert lib.gq_matvec_id_workspace(128, 8, 8, 704, ctypes.byref(need)) == GQ_OK
    assert call(a15=need.value - 1) == GQ_ERR_WORKSPACE
    assert call(a7=0, a1=None, a2=None, a6=None, a9=None, a12=None, a14=None) == GQ_OK  # no tokens: no-op
    assert call(a4=0) == GQ_OK  # N == 0: no-op


def test_matvec_id_noalloc_validation(lib):
    """The no-allocation routed product validates like gq_matvec_id and refuses
    a call whose workspace would exceed its per-GPU array (8 MiB), all on the
    host, before any HIP call."""
    f = lib.gq_matvec_id_noalloc
    args = [1, A, 128, 704, 2816, A, 8, 8, A, 0, 0, None, A, None]
    names = ["t", "ex", "E", "N", "K", "ids", "T", "k", "x", "xd", "per", "rw", "y", "s"]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(t=5) == GQ_ERR_TYPE
    assert call(xd=2) == GQ_ERR_DTYPE
    assert call(K=2817) == GQ_ERR_SHAPE
    assert call(T=129) == GQ_ERR_SHAPE
    assert call(ids=None, y=None) == GQ_ERR_NULL
    assert call(y=None) == GQ_ERR_NULL
    assert call(y=MIS) == GQ_ERR_ALIGN
    assert call(ids=MIS) == GQ_ERR_ALIGN
    # 1024 slots of N = 2816: 11.5 MB of per-slot outputs for a weighted call
    assert call(T=128, rw=A, N=2816, K=704) == GQ_ERR_WORKSPACE
    sz = ctypes.c_size_t()
    assert lib.gq_matvec_id_workspace(128, 128, 8, 2816, ctypes.byref(sz)) == GQ_OK and sz.value > 8 << 20
    assert call(T=0) == GQ_OK  # no tokens: no-op


def test_route_topk_plan_validation(lib):
    f = lib.gq_route_topk_plan
    sz = ctypes.c_size_t()
    assert lib.gq_matvec_id_workspace(128, 8, 8, 0, ctypes.byref(sz)) == GQ_OK
    need = sz.value
    ok = [A, 8, 128, 8, A, A, A, need, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a3=0) == GQ_ERR_SHAPE
    assert call(a3=129) == GQ_ERR_SHAPE      # top_k > n_experts
    assert call(a1=129) == GQ_ERR_SHAPE      # 129 * 8 slots > 1024
    assert call(a2=5000, a1=1) == GQ_ERR_UNSUPPORTED
    for i in (0, 4, 5, 6):
        assert call(**{"a%d" % i: None}) == GQ_ERR_NULL, i
        assert call(**{"a%d" % i: MIS}) == GQ_ERR_ALIGN, i
    assert call(a7=need - 1) == GQ_ERR_WORKSPACE
    assert call(a1=0, a0=None, a4=None, a5=None, a6=None) == GQ_OK  # no tokens: no-op


def test_route_matvec_id_glu_validation(lib):
    """Routing and the routed gated unit in one call: the union of the router's
    and the gated unit's checks, all on the host."""
    f = lib.gq_route_matvec_id_glu
    need = ctypes.c_size_t()
    assert lib.gq_matvec_id_workspace(128, 8, 8, 704, ctypes.byref(need)) == GQ_OK
    # (type, gate, up, n_experts, N, K, logits, n_tokens, top_k, ids, weights, x, x_dtype, act, h, h_dtype, ws,
    #  ws_bytes, stream)
    ok = [1, A, A, 128, 704, 2816, A, 8, 8, A, A, A, 0, 0, A, 1, A, need.value, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a0=9) == GQ_ERR_TYPE
    assert call(a12=2) == GQ_ERR_DTYPE  # fp16 activations
    assert call(a15=2) == GQ_ERR_DTYPE  # fp16 output
    assert call(a5=100) == GQ_ERR_SHAPE  # K not whole blocks
    assert call(a3=0) == GQ_ERR_SHAPE
    assert call(a8=0) == GQ_ERR_SHAPE
    assert call(a8=129) == GQ_ERR_SHAPE  # top_k > n_experts
    assert call(a7=129) == GQ_ERR_SHAPE  # 129 * 8 slots > 1024
    assert call(a3=5000, a7=1) == GQ_ERR_UNSUPPORTED  # more experts than the router takes
    assert call(a13=2) == GQ_ERR_UNSUPPORTED  # unknown activation
    for i in (1, 2, 6, 9, 10, 11, 14, 16):
        assert call(**{"a%d" % i: None}) == GQ_ERR_NULL, i
        assert call(**{"a%d" % i: MIS}) == GQ_ERR_ALIGN, i
    assert call(a17=need.value - 1) == GQ_ERR_WORKSPACE
    assert call(a7=0, a1=None, a2=None, a6=None, a9=None, a10=None, a11=None, a14=None, a16=None) == GQ_OK
