"""Build libgq.so (the C ABI in include/gq.h) for gfx950 with hipcc.

    python -m block_quantized_weight_q4_amd.build

Every HIP/C++ source under csrc/ is compiled in parallel into _build/ and
linked into block_quantized_weight_q4_amd/libgq.so; floor/gq_floor.hip (the
plain streaming read the benchmark reports against, not part of the C ABI)
becomes libgqfloor.so.  The build always recompiles (it is the "does it
build" check), using an atomic rename so a loaded copy is never overwritten
in place.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libgq.so")
FLOOR_SRC = os.path.join(PKG, "floor", "gq_floor.hip")
FLOOR_OUT = os.path.join(PKG, "libgqfloor.so")
BUILD = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # never let the compiler form packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs) + 1, max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        floor_obj = ex.submit(_compile, FLOOR_SRC)
        objs = list(ex.map(_compile, srcs))
        _link([floor_obj.result()], FLOOR_OUT)
    _link(objs, OUT)
    if verbose:
        print("built", OUT, "and", FLOOR_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
