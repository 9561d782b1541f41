"""Benchmark of the packed-weight products on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu-baseline]
    python bench.py --context-only        (the context workloads alone, for kernel traces)
    python bench.py --floor-only          (the stream-read kernel at the headline's byte counts)
    python bench.py --pmc-pass            (the dominant kernel + a copy kernel, for rocprofv3 --pmc)
    python bench.py --prefill-pass        (the Q4_K prefill product alone, for rocprofv3 --pmc)
    python bench.py --traffic-summary FETCH_DIR WRITE_DIR   (writes profiles/<kernel>_traffic.txt)
    python bench.py --mfma-summary DIR                      (writes profiles/<prefill>_mfma_counters.txt)
    python bench.py --stats-summary DIR OUT.txt             (rocprofv3 --stats CSV -> text summary)
    python bench.py --abba LIB_A LIB_B [--rounds R] [--workload headline|moe|prefill]
                                          (two builds of libgq.so compared A-B-B-A in fresh processes)

The step (the headline workload) is one decoder layer of Q4_K products at
batch 1, hidden 2560: q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up
9728x2560, down 2560x9728 -- 56,770,560 packed bytes.  q|k|v and gate|up read
the same activation vector and are issued as one launch each over their
row-concatenated weights (a loader stores them that way), so a step is four
dependent launches: qkv, o, gate|up, down.  The launches are the list
block_quantized_weight_q4_amd.workloads.HEADLINE, which the parity tests walk
too.  Weights rotate over >= 1 GiB of distinct copies so each step streams
from HBM, not from the 256 MB last-level cache; inputs are resident in HBM
before the timed region.  The steps are captured once in a HIP graph that
walks every copy; the timed region replays it at least 5 times (more when
--steps asks for more steps), each replay between its own HIP events on the
launch stream, bracketed by device synchronisation.

One JSON line: value = packed-weight GB/s of the whole step (total bytes of
all timed steps / total time), with the median and minimum per replay;
`launches` = each of the four launches alone, against the time of a plain
streaming read of the same number of bytes (libgqfloor.so, measured in the
same run); roofline = the dominant kernel (gate|up, 28,016,640 B per launch)
timed over back-to-back launches of it alone; cpu_baseline = the CPU oracle on
the same layer, on all the host cores the process may use (one thread per
core, over row ranges) and on one; plus the prefill products' TFLOP/s and the
other workloads as context.

roofline.traffic is the HBM bytes per launch of that kernel from two
rocprofv3 --pmc runs of `--pmc-pass` (FETCH_SIZE, then WRITE_SIZE), each
scaled by the factor that makes the same counter read right for a plain copy
kernel of known size.  prefill.mfma_busy comes from one rocprofv3 --pmc run of
`--prefill-pass`.  Each summary file records a hash of the kernel's sources;
when the sources have changed since, the figure is reported as null.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_quantized_weight_q4_amd import workloads as WL  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "packed-weight GB/s (% of HBM peak), Q4_K GEMV batch 1; prefill TFLOP/s"
ROTATE_BYTES = 1 << 30
MIN_REPS = 5
CSRC = os.path.join(ROOT, "block_quantized_weight_q4_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline only (no context workloads)")
    ap.add_argument("--context-only", action="store_true",
                    help="only the context workloads (one JSON line of them; for kernel traces)")
    ap.add_argument("--floor-only", action="store_true", help="only the stream-read kernel at the headline sizes")
    ap.add_argument("--pmc-pass", action="store_true", help="run the dominant kernel 8x and one copy kernel")
    ap.add_argument("--pmc-moe-pass", metavar="META_JSON",
                    help="run the fused MoE layer (8 and 64 tokens, 3 times each) and one copy kernel; "
                         "writes each layer's routing facts to META_JSON")
    ap.add_argument("--moe-traffic-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "META_JSON"))
    ap.add_argument("--prefill-pass", action="store_true", help="run the Q4_K prefill product a few times")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--mfma-summary", metavar="DIR")
    ap.add_argument("--stats-summary", nargs=2, metavar=("DIR", "OUT"))
    ap.add_argument("--abba", nargs=2, metavar=("LIB_A", "LIB_B"))
    ap.add_argument("--rounds", type=int, default=4, help="A-B-B-A blocks for --abba")
    ap.add_argument("--workload", default="headline", help="workload --abba / --measure-only time")
    ap.add_argument("--measure-only", action="store_true", help="time --workload alone (one JSON line)")
    return ap.parse_args()


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ traffic
DOM = WL.DOMINANT
GU_KERNEL = "k_matvec<2, 0, 1"          # Q4_K, fp32 activations, batch 1
COPY_BYTES = 64 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "matvec_q4k_gateup_19456x2560_b1_traffic.txt")
KERNEL_SOURCES = ["gq_device.h", "gq_gemv_core.h", "gq_matvec.hip"]
PREFILL = WL.TIMED_MATMUL[0]
MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_q4k_3015x17408x5120_mfma_counters.txt")
MOE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_q4_0_128x_h2816_f704_top8_traffic.txt")
MOE_SOURCES = ["gq_device.h", "gq_gemv_core.h", "gq_route_core.h", "gq_matvec_id.hip"]
MFMA_SOURCES = ["gq_device.h", "gq_matmul.hip"]
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16"]


def pmc_pass():
    """The dominant kernel (gate|up, batch 1) over 8 distinct weight copies,
    then torch's elementwise add over a 64 MiB fp32 tensor: 64 MiB read,
    64 MiB written, the calibration for the byte counters."""
    import torch
    import block_quantized_weight_q4_amd as gq
    dev = torch.device("cuda:0")
    W = DOM.weight()
    Ws = [torch.from_numpy(W).to(dev) for _ in range(8)]
    x = torch.from_numpy(DOM.x()).to(dev)
    y = torch.empty(1, DOM.N, device=dev)
    for w in Ws:
        gq.gq_matvec(DOM.t, w, DOM.N, DOM.K, x, y)
    torch.cuda.synchronize()
    src = torch.empty(COPY_BYTES // 4, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    print("pmc pass done", flush=True)


def pmc_moe_pass(meta_path: str):
    """The fused MoE layer (router and gated unit, weighted down product on
    the group table they leave) on one copy of the experts, 3 times at 8 tokens and
    3 times at 64 tokens (top 8 of 128), then the copy kernel of pmc_pass.
    meta_path gets, per layer in launch order, the token count, the distinct
    experts the router chose, the group count of the table and the bytes of
    one expert matrix, for --moe-traffic-summary."""
    import torch
    import block_quantized_weight_q4_amd as gq
    dev = torch.device("cuda:0")
    base = WL.MOE
    ex = {k: torch.from_numpy(v).to(dev) for k, v in base.experts().items()}
    meta = []
    for T in (8, 64):
        m = WL.MoeLayer(T=T)
        lg = torch.from_numpy(m.logits()).to(dev)
        x = torch.from_numpy(m.x()).to(dev)
        ids = torch.empty((T, m.k), dtype=torch.int32, device=dev)
        rw = torch.empty((T, m.k), device=dev)
        hb = torch.empty((T, m.k, m.F), device=dev, dtype=torch.bfloat16)
        yd = torch.empty(T, m.H, device=dev)
        ws = torch.zeros(gq.gq_matvec_id_workspace(m.E, T, m.k, m.H), dtype=torch.uint8, device=dev)
        for _ in range(3):
            gq.gq_route_matvec_id_glu(m.t, ex["gate"], ex["up"], m.E, m.F, m.H, lg, m.k, ids, rw, x, "silu", hb, ws)
            gq.gq_matvec_id(m.t, ex["down"], m.E, m.H, m.F, (T, m.k), hb, True, yd, ws, rw)
            torch.cuda.synchronize()
            hdr = ws[:8].view(torch.int32).cpu().numpy()
            _, counts = np.unique(ids.cpu().numpy(), return_counts=True)
            # groups of at most 8 slots per expert (the table of the one-launch
            # form is indexed by slot, so its header holds the slot count)
            groups = int(sum((c + 7) // 8 for c in counts))
            meta.append({"tokens": T, "top_k": m.k, "experts": m.E, "distinct_experts": int(counts.size),
                         "groups": groups, "invalid_ids": int(hdr[0]),
                         "expert_matrix_bytes": int(ex["down"].numel() // m.E)})
    src = torch.empty(COPY_BYTES // 4, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    with open(meta_path, "w") as f:
        json.dump(meta, f)
    print("moe pmc pass done", flush=True)


def moe_traffic_summary(fetch_dir: str, write_dir: str, meta_path: str):
    """HBM bytes of each fused MoE layer of --pmc-moe-pass (the sum over its
    router, gated-unit and down-product dispatches, FETCH_SIZE and WRITE_SIZE
    scaled by the copy kernel's calibration) against the bytes of the expert
    matrices it had to read: once per distinct expert, and once per group of
    the table (an expert with more than 8 slots is read once per 8)."""
    import csv
    import glob
    meta = json.load(open(meta_path))
    per_ctr = {}
    for d, ctr in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        runs = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True),
                      key=os.path.getmtime)
        rows = [r for r in csv.DictReader(open(runs[-1])) if r["Counter_Name"] == ctr]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        cp = [float(r["Counter_Value"]) for r in rows
              if "vectorized_elementwise_kernel" in r["Kernel_Name"] and "add" in r["Kernel_Name"].lower()]
        assert len(cp) == 1, cp
        factor = (COPY_BYTES / 1024.0) / cp[0]
        # a layer starts with the routing launch: the routed gated unit (8
        # tokens) or the router with its table (64 tokens)
        layers, cur = [], None
        for r in rows:
            name = r["Kernel_Name"]
            if "k_route_plan" in name or "k_experts_routed" in name:
                cur = []
                layers.append(cur)
            if cur is not None and ("k_route_plan" in name or "k_experts" in name):
                cur.append(float(r["Counter_Value"]) * 1024.0 * factor)
        assert len(layers) == len(meta) and all(len(l) in (2, 3) for l in layers), (
            len(layers), [len(l) for l in layers])
        per_ctr[ctr] = (layers, factor)
    out = ["# HBM traffic of the fused MoE layer (128 Q4_0 experts, hidden 2816, FFN 704, top 8) at 8 and 64 tokens",
           "",
           "kernels: 8 tokens: k_experts_routed (routing + gate|up + SiLU, bf16 h), then the weighted down",
           "product k_experts on the table it leaves; 64 tokens: k_route_plan (router + group table), the",
           "k_experts GLU form, the weighted down product on that table; one copy of the experts, so every",
           "layer reads its experts from HBM or the last-level cache, not from L2 (4 MB per XCD)",
           "source_sha256: %s" % source_hash(MOE_SOURCES),
           "commands (from the repository root, on the GPU host):",
           "  timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -- python3 bench.py "
           "--pmc-moe-pass <DIR>/meta_fetch.json",
           "  timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -- python3 bench.py "
           "--pmc-moe-pass <DIR>/meta_write.json",
           "  python bench.py --moe-traffic-summary <FETCH_DIR> <WRITE_DIR> <DIR>/meta_fetch.json",
           "",
           "calibration (copy kernel of %d MiB): FETCH_SIZE x %.3f, WRITE_SIZE x %.3f"
           % (COPY_BYTES >> 20, per_ctr["FETCH_SIZE"][1], per_ctr["WRITE_SIZE"][1]),
           "",
           "%-7s %9s %7s %14s %14s %14s %9s %9s" % ("tokens", "distinct", "groups", "read_bytes", "distinct_bytes",
                                                     "group_bytes", "read/dist", "read/grp")]
    for i, m in enumerate(meta):
        fetch = sum(per_ctr["FETCH_SIZE"][0][i])
        mb = m["expert_matrix_bytes"]
        dist_b = 3 * mb * m["distinct_experts"]
        grp_b = 3 * mb * m["groups"]
        out.append("%-7d %9d %7d %14.0f %14d %14d %9.4f %9.4f" % (m["tokens"], m["distinct_experts"], m["groups"],
                                                                  fetch, dist_b, grp_b, fetch / dist_b,
                                                                  fetch / grp_b))
    out += ["", "read_bytes: FETCH_SIZE of the layer's routing and product dispatches (weights, activations, logits,",
            "the table);",
            "written bytes per layer (WRITE_SIZE): " + ", ".join(
                "%.0f" % sum(l) for l in per_ctr["WRITE_SIZE"][0])]
    with open(MOE_TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def prefill_pass():
    """The Q4_K prefill product 5 times (the counters of each dispatch are
    averaged by the summary)."""
    import torch
    import block_quantized_weight_q4_amd as gq
    dev = torch.device("cuda:0")
    L = PREFILL
    W = torch.from_numpy(L.weight()).to(dev)
    X = torch.from_numpy(L.x_bf16_bits().view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty(L.M, L.N, device=dev)
    for _ in range(5):
        gq.gq_matmul(L.t, W, L.N, L.K, X, Y)
    torch.cuda.synchronize()
    print("prefill pass done", flush=True)


def _counter_means(d: str) -> tuple[dict, dict]:
    import csv
    import glob
    vals = {}
    # the newest run in the directory only
    runs = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True), key=os.path.getmtime)
    for p in runs[-1:]:
        for r in csv.DictReader(open(p)):
            vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def traffic_summary(fetch_dir: str, write_dir: str):
    out_lines = []
    per = {}
    kname = ""
    for d, ctr in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        means, counts = _counter_means(d)
        mv = [k for k in means if k[1] == ctr and GU_KERNEL in k[0]]
        cp = [k for k in means if k[1] == ctr and "vectorized_elementwise_kernel" in k[0] and "add" in k[0].lower()]
        assert len(mv) == 1 and len(cp) == 1, (mv, cp)
        kib_mv, kib_cp = means[mv[0]], means[cp[0]]
        factor = (COPY_BYTES / 1024.0) / kib_cp
        per[ctr] = (kib_mv, kib_cp, factor, counts[mv[0]])
        kname = mv[0][0]
        out_lines.append("%s: dominant kernel %.1f KiB/dispatch (mean of %d); copy kernel %.1f KiB for %d KiB "
                         "moved -> scale %.4f -> %.0f bytes per launch"
                         % (ctr, kib_mv, counts[mv[0]], kib_cp, COPY_BYTES // 1024, factor, kib_mv * factor * 1024))
    traffic = sum(v[0] * v[2] * 1024 for v in per.values())
    algo = DOM.N * (DOM.K // 256) * 144
    text = ["# HBM traffic of the Q4_K gate|up product (19456 x 2560, batch 1, fp32 x)",
            "",
            "kernel: %s (Q4_K, fp32 activations, batch 1)" % kname.split("(unsigned")[0].replace("void ", ""),
            "source_sha256: %s" % source_hash(KERNEL_SOURCES),
            "commands (from the repository root, on the GPU host):",
            "  timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -- python3 bench.py --pmc-pass",
            "  timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -- python3 bench.py --pmc-pass",
            "  python bench.py --traffic-summary <FETCH_DIR> <WRITE_DIR>",
            ""] + out_lines + [
            "",
            "traffic_bytes_per_launch: %.0f" % traffic,
            "algorithmic_bytes_per_launch: %d (packed weights) + %d (x) + %d (y)" % (algo, DOM.K * 4, DOM.N * 4),
            "traffic / algorithmic: %.4f" % (traffic / (algo + DOM.K * 4 + DOM.N * 4))]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def _short_kernel_name(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0]


def mfma_summary(d: str):
    """Matrix-core utilisation of the prefill kernel from one counter pass.

    SQ_VALU_MFMA_BUSY_CYCLES is summed over every SIMD of the chip (it equals
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops / 1024 flops per SIMD cycle, the
    bf16 rate of one SIMD), and GRBM_GUI_ACTIVE over the 8 XCDs.  The cycles
    the matrix cores could have worked are therefore
    GRBM_GUI_ACTIVE / 8 x 1024 SIMDs, and the utilisation is the ratio.  It is
    counted in the clock the chip ran at, which under this load is below the
    2.4 GHz of the published peak; the time the kernel takes gives that clock."""
    means, counts = _counter_means(d)
    ks = sorted({k[0] for k in means if "k_matmul" in k[0]})
    assert len(ks) >= 1, ks
    kname = ks[0]
    v = {c: means.get((kname, c)) for c in MFMA_COUNTERS}
    n = counts.get((kname, MFMA_COUNTERS[0]), 0)
    xcds, simds = 8, 1024
    cycles = v["GRBM_GUI_ACTIVE"] / xcds
    util = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * simds) if cycles else float("nan")
    flops = v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    text = ["# MFMA counters of the Q4_K prefill product (%d x %d x %d, bf16 activations)" % (PREFILL.M, PREFILL.N,
                                                                                           PREFILL.K),
            "",
            "kernel: %s" % _short_kernel_name(kname),
            "source_sha256: %s" % source_hash(MFMA_SOURCES),
            "command (from the repository root, on the GPU host):",
            "  timeout -s KILL 60 rocprofv3 --pmc %s --output-format csv -d <DIR> -- python3 bench.py --prefill-pass"
            % " ".join(MFMA_COUNTERS),
            "  python bench.py --mfma-summary <DIR>",
            "",
            "dispatches averaged: %d" % n] + ["%s: %.6g" % (c, v[c]) for c in MFMA_COUNTERS] + [
            "",
            "MFMA flops per dispatch (MOPS x 512): %.4g (2 x M x N x K with M padded to whole 256-row tiles: %.4g)"
            % (flops, 2.0 * -(-PREFILL.M // 256) * 256 * PREFILL.N * PREFILL.K),
            "kernel cycles (GRBM_GUI_ACTIVE / %d XCDs): %.4g" % (xcds, cycles),
            "mfma_busy_fraction: %.4f   (SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x %d SIMDs))" % (util, simds)]
    with open(MFMA_FILE, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def read_summary(path: str, key: str, sources) -> float | None:
    """A figure from a committed summary, or None when the kernel sources
    changed since it was taken (or there is none)."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"source_sha256: (\w+)", text)
    t = re.search(key + r": ([0-9.eE+-]+)", text)
    if not m or not t or m.group(1) != source_hash(sources):
        return None
    return float(t.group(1))


def stats_summary(d: str, out: str):
    """rocprofv3 --kernel-trace --stats output -> short text table."""
    import csv
    import glob
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    assert stats and trace, d
    lines = ["%-100s %7s %10s %10s %10s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
    for r in csv.DictReader(open(stats[0])):
        lines.append("%-100s %7s %10.3f %10.3f %10.3f" % (r["Name"][:100], r["Calls"], float(r["AverageNs"]) / 1e3,
                                                      float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    # per (kernel, grid) averages from the trace: one kernel serves several shapes
    per = {}
    for r in csv.DictReader(open(trace[0])):
        gy = int(r.get("Grid_Size_Y") or 1)
        grid = r["Grid_Size_X"] if gy == 1 else "%sx%d" % (r["Grid_Size_X"], gy)
        k = (r["Kernel_Name"][:80], grid, int(r["Workgroup_Size_X"]))
        per.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "per launch shape (grid = work-items, x or x by y):",
              "%-80s %11s %5s %7s %10s %10s" % ("kernel", "grid", "wg", "calls", "avg_us", "median_us")]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        lines.append("%-80s %11s %5d %7d %10.3f %10.3f" % (k[0], k[1], k[2], len(v), sum(v) / len(v), v[len(v) // 2]))
    with open(out, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------ timing
class Timer:
    """Capture a list of launches once in a HIP graph; replay and time it."""

    def __init__(self, torch, fn, stream):
        self.torch, self.fn, self.stream = torch, fn, stream
        fn()  # warm the code objects before capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=stream):
            fn()
        torch.cuda.synchronize()

    def replays(self, reps: int, warm: int = 2) -> list[float]:
        """ms of each of `reps` back-to-back replays (events between them on
        the launch stream, no host synchronisation until the last)."""
        torch = self.torch
        for _ in range(warm):
            self.graph.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(self.stream)
        for i in range(reps):
            self.graph.replay()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]

    def time(self, reps: int, warm: int = 2) -> float:
        """Mean ms per replay over `reps` replays."""
        r = self.replays(reps, warm)
        return sum(r) / len(r)


def eager_ms(torch, fn, stream, reps: int = 30, warm: int = 60) -> list[float]:
    """ms of each of `reps` back-to-back eager calls of fn on `stream` (events
    between them), for library calls that are not captured in a graph."""
    with torch.cuda.stream(stream):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def n_copies(nbytes: int) -> int:
    return max(2, -(-ROTATE_BYTES // nbytes))


class Floor:
    """The plain streaming read (libgqfloor.so) at a given byte count, over
    rotated buffers like the products it is compared with."""

    def __init__(self, torch, stream):
        path = os.path.join(ROOT, "block_quantized_weight_q4_amd", "libgqfloor.so")
        if not os.path.exists(path):
            raise RuntimeError("libgqfloor.so is not built (python -m block_quantized_weight_q4_amd.build)")
        self.lib = ctypes.CDLL(path)
        self.lib.gqf_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_void_p]
        self.lib.gqf_stream_read.restype = ctypes.c_int
        self.torch, self.stream = torch, stream
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def us(self, nbytes: int, reps: int = MIN_REPS) -> float:
        torch = self.torch
        nb = (nbytes + 15) // 16 * 16
        bufs = [torch.full((nb,), 1, dtype=torch.uint8, device="cuda") for _ in range(n_copies(nb))]
        threads = 512 if nb >= (20 << 20) else 256

        def run():
            for b in bufs:
                rc = self.lib.gqf_stream_read(b.data_ptr(), nb, self.sink.data_ptr(), threads, self.stream.cuda_stream)
                if rc:
                    raise RuntimeError("gqf_stream_read failed: %d" % rc)

        r = Timer(torch, run, self.stream).replays(reps)
        del bufs
        torch.cuda.empty_cache()
        return float(np.median(r)) * 1e3 / n_copies(nb)


def floor_only(torch, stream):
    fl = Floor(torch, stream)
    out = {}
    for L in WL.HEADLINE:
        nb = L.N * (L.K // 256) * 144
        out[L.name] = {"bytes": nb, "floor_us": round(fl.us(nb), 3)}
        print("floor %s %d B: %.3f us" % (L.name, nb, out[L.name]["floor_us"]), flush=True)
    lb = WL.layer_bytes("dense")
    out["layer_as_one_read"] = {"bytes": lb, "floor_us": round(fl.us(lb), 3)}
    print(json.dumps({"stream_floor": out}))


# ------------------------------------------------------------ main
def main():
    args = parse()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    if args.mfma_summary:
        return mfma_summary(args.mfma_summary)
    if args.stats_summary:
        return stats_summary(*args.stats_summary)
    if args.abba:
        return abba(*args.abba, rounds=args.rounds, workload=args.workload)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the products shard by "
              "output rows across GPUs).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.pmc_pass:
        return pmc_pass()
    if args.pmc_moe_pass:
        return pmc_moe_pass(args.pmc_moe_pass)
    if args.moe_traffic_summary:
        return moe_traffic_summary(*args.moe_traffic_summary)
    if args.prefill_pass:
        return prefill_pass()

    import torch
    import block_quantized_weight_q4_amd as gq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    side = torch.cuda.Stream()  # graphs are captured on a non-default stream
    torch.cuda.set_stream(side)
    stream = torch.cuda.current_stream()

    def t_(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if args.floor_only:
        return floor_only(torch, stream)
    if args.measure_only:
        print(json.dumps({"workload": args.workload,
                          "ms_per_step": measure(torch, gq, dev, stream, t_, args.workload)}), flush=True)
        return
    if args.context_only:
        print(json.dumps({"context": bench_context(torch, gq, dev, stream, t_)}), flush=True)
        return

    # ------------------------------------------------ headline: dense layer
    launches = WL.HEADLINE
    host = {L.name: L.weight() for L in launches}
    layer_bytes = WL.layer_bytes("dense")
    assert layer_bytes == sum(w.nbytes for w in host.values())
    nc = n_copies(layer_bytes)
    copies = [{k: t_(v) for k, v in host.items()} for _ in range(nc)]
    xs = {L.name: t_(L.x()) for L in launches}
    ys = {L.name: torch.empty(1, L.N, device=dev) for L in launches}

    def layer_pass():
        for c in copies:
            for L in launches:
                gq.gq_matvec(L.t, c[L.name], L.N, L.K, xs[L.name], ys[L.name], stream)

    tl = Timer(torch, layer_pass, stream)
    reps = max(MIN_REPS, math.ceil(args.steps / nc))
    warm = max(2, math.ceil(args.warmup / nc))
    torch.cuda.synchronize()
    rep_ms = tl.replays(reps, warm)
    torch.cuda.synchronize()
    steps = reps * nc
    ms_step = sum(rep_ms) / steps
    per_rep = sorted(r / nc for r in rep_ms)
    value = layer_bytes / (ms_step * 1e-3) / 1e9
    del tl

    # each launch alone, back to back over the copies, and the stream floor
    # of its byte count
    fl = Floor(torch, stream)
    per_launch = {}
    for L in launches:
        def one(L=L):
            for c in copies:
                gq.gq_matvec(L.t, c[L.name], L.N, L.K, xs[L.name], ys[L.name], stream)

        r = sorted(v / nc * 1e3 for v in Timer(torch, one, stream).replays(MIN_REPS))
        nb = host[L.name].nbytes
        f_us = fl.us(nb)
        per_launch[L.name] = {"shape": "%dx%d" % (L.N, L.K), "bytes": nb, "us_median": round(r[len(r) // 2], 3),
                              "us_min": round(r[0], 3), "floor_us": round(f_us, 3),
                              "pct_of_floor": round(100.0 * f_us / r[len(r) // 2], 1),
                              "pct_hbm_peak": round(100.0 * nb / (r[len(r) // 2] * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
    floor_sum = sum(v["floor_us"] for v in per_launch.values())
    peak_read = fl.us(1 << 29, reps=3)
    read_peak_gbs = (1 << 29) / (peak_read * 1e-6) / 1e9

    # dominant kernel: gate|up alone, back to back over the copies
    gu_us = per_launch[DOM.name]["us_median"]
    gu_mean_ms = None

    def gu_pass():
        for c in copies:
            gq.gq_matvec(DOM.t, c[DOM.name], DOM.N, DOM.K, xs[DOM.name], ys[DOM.name], stream)

    tg = Timer(torch, gu_pass, stream)
    gu_mean_ms = tg.time(max(MIN_REPS, reps)) / nc
    gu_bytes = host[DOM.name].nbytes

    # the same launches with their weights already in a cache: the whole
    # layer alternating over two copies (113 MB: above the 8 x 4 MB of L2,
    # inside the 256 MB last-level cache) and gate|up on one copy (28 MB,
    # spread over the XCDs' L2s).  Context for the fixed cost per launch: a
    # launch bound by HBM alone would shrink with its bytes' source.
    def warm_layer():
        for i in range(nc):
            for L in launches:
                gq.gq_matvec(L.t, copies[i % 2][L.name], L.N, L.K, xs[L.name], ys[L.name], stream)

    def warm_gu():
        for _ in range(nc):
            gq.gq_matvec(DOM.t, copies[0][DOM.name], DOM.N, DOM.K, xs[DOM.name], ys[DOM.name], stream)

    cache_warm = {
        "layer_us_from_last_level_cache": round(float(np.median(Timer(torch, warm_layer, stream).replays(MIN_REPS)))
                                                * 1e3 / nc, 2),
        "gate_up_us_from_l2": round(float(np.median(Timer(torch, warm_gu, stream).replays(MIN_REPS))) * 1e3 / nc, 3),
        "layer_us_from_hbm": round(per_rep[len(per_rep) // 2] * 1e3, 2),
        "gate_up_us_from_hbm": gu_us,
    }
    gu_gbs = gu_bytes / (gu_mean_ms * 1e-3) / 1e9
    del tg, copies
    torch.cuda.empty_cache()

    # ------------------------------------------------ prefill products
    prefill = None
    others = {}
    for L in WL.TIMED_MATMUL:
        W5 = t_(L.weight())
        X5 = t_(L.x_bf16_bits().view(np.int16)).view(torch.bfloat16)
        Y5 = torch.empty(L.M, L.N, device=dev)
        tp = Timer(torch, lambda: gq.gq_matmul(L.t, W5, L.N, L.K, X5, Y5, stream), stream)
        # the matrix cores reach their sustained clock only after some tens of
        # milliseconds of this load: replay well past that before timing
        r = sorted(tp.replays(30, warm=60))
        ms_mm = float(np.median(r))
        flops = 2.0 * L.M * L.N * L.K
        tf = flops / (ms_mm * 1e-3) / 1e12
        if L is PREFILL:
            prefill = {"workload": "q4_k_prefill_%dx%dx%d_bf16" % (L.M, L.N, L.K), "ms": round(ms_mm, 4),
                       "ms_min": round(r[0], 4), "TFLOPs": round(tf, 2),
                       "frac_bf16_dense_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                       "mfma_busy_fraction": read_summary(MFMA_FILE, "mfma_busy_fraction", MFMA_SOURCES),
                       "tokens_per_s": round(L.M / (ms_mm * 1e-3), 1)}
            # context: the same product with all-zero activations (the time
            # depends on the data when the chip runs at its power limit), and
            # the vendor's plain bf16 GEMM (torch.matmul -> hipBLASLt, weights
            # already dense bf16, bf16 output) at this shape
            X0 = torch.zeros_like(X5)
            t0 = Timer(torch, lambda: gq.gq_matmul(L.t, W5, L.N, L.K, X0, Y5, stream), stream)
            ms_zero = float(np.median(t0.replays(30, warm=60)))
            del t0, X0
            gen = torch.Generator(device=dev)
            gen.manual_seed(WL.S_PREFILL + 1000)
            WT = torch.randn(L.K, L.N, device=dev, generator=gen).to(torch.bfloat16).contiguous()
            ms_blas = float(np.median(eager_ms(torch, lambda: torch.matmul(X5, WT), stream)))
            del WT
            prefill["context"] = {
                "ms_with_zero_activations": round(ms_zero, 4),
                "vendor_bf16_gemm": {"what": "torch.matmul(X bf16 [M,K], W^T bf16 [K,N]) -> bf16 (hipBLASLt), "
                                             "random weights, eager, median of 30 after 60 warm-up calls",
                                     "ms": round(ms_blas, 4),
                                     "TFLOPs": round(flops / (ms_blas * 1e-3) / 1e12, 2),
                                     "fused_q4_k_over_vendor_bf16": round(ms_blas / ms_mm, 4)}}
        else:
            others["%s_prefill_%dx%dx%d_bf16" % (L.t, L.M, L.N, L.K)] = {"ms": round(ms_mm, 4),
                                                                         "TFLOPs": round(tf, 2)}
        del tp, W5, X5, Y5
        torch.cuda.empty_cache()
    prefill["other_formats"] = others

    context = {} if args.quick else bench_context(torch, gq, dev, stream, t_)

    # ------------------------------------------------ CPU oracle on the host
    cpu = None if args.no_cpu_baseline else cpu_baseline(launches, host, xs)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(per_rep[len(per_rep) // 2], 5),
        "ms_per_step_min": round(per_rep[0], 5),
        "timed_replays": reps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32",
        "data": "synthetic",
        "config": {
            "workload": "q4_k_gemv_dense_layer_hidden2560_batch1",
            "layer": "q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up 9728x2560, down 2560x9728 (Q4_K)",
            "launches_per_step": "qkv 6144x2560, o, gate|up 19456x2560, down (HIP graph)",
            "batch": 1,
            "packed_bytes_per_step": layer_bytes,
            "weight_copies_rotated": nc,
            "activations": "fp32 N(0,1)",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "pct_of_measured_read_peak": round(100.0 * value / read_peak_gbs, 2),
        "tokens_per_s_equiv": round(value / 2.74, 1),
        "launches": per_launch,
        "stream_floor": {"kernel": "k_stream_read (one 16-byte load per work-item, libgqfloor.so)",
                         "sum_of_launch_floors_us": round(floor_sum, 3),
                         "pct_of_floor": round(100.0 * floor_sum / (ms_step * 1e3), 1),
                         "read_peak_GBs_512MiB": round(read_peak_gbs, 1)},
        "cache_warm": cache_warm,
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                     "traffic": read_summary(TRAFFIC_FILE, "traffic_bytes_per_launch", KERNEL_SOURCES),
                     "kernel": "k_matvec<Q4_K, fp32, batch 1> gate|up 19456x2560",
                     "bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_mean_ms * 1e3, 3),
                     "median_launch_us": gu_us},
        "cpu_baseline": cpu,
        "prefill": prefill,
        "context": context,
    }
    print(json.dumps(out))


def measure(torch, gq, dev, stream, t_, workload: str) -> float:
    """ms per step of one workload, timed as in the full run (median of the
    replays; the headline and MoE layers over rotated weight copies)."""
    if workload == "headline":
        launches = WL.HEADLINE
        host = {L.name: L.weight() for L in launches}
        nc = n_copies(WL.layer_bytes("dense"))
        cps = [{k: t_(v) for k, v in host.items()} for _ in range(nc)]
        xs = {L.name: t_(L.x()) for L in launches}
        ys = {L.name: torch.empty(1, L.N, device=dev) for L in launches}

        def run():
            for c in cps:
                for L in launches:
                    gq.gq_matvec(L.t, c[L.name], L.N, L.K, xs[L.name], ys[L.name], stream)

        return float(np.median(Timer(torch, run, stream).replays(2 * MIN_REPS))) / nc
    if workload in ("moe", "moe:64", "moe:split"):
        # the fused MoE layer at 8 tokens ("moe", the context workload) or 64;
        # "moe:split": at 8 tokens with the router and its table in a launch
        # of their own before the gated unit
        m = WL.MoeLayer(T=64) if workload == "moe:64" else WL.MOE
        split = workload == "moe:split"
        ex = m.experts()
        nb = sum(v.nbytes for v in ex.values())
        cps = [{k: t_(v) for k, v in ex.items()} for _ in range(n_copies(nb))]
        lg, x4 = t_(m.logits()), t_(m.x())
        ids = torch.empty((m.T, m.k), dtype=torch.int32, device=dev)
        rw = torch.empty((m.T, m.k), device=dev)
        hb = torch.empty((m.T, m.k, m.F), device=dev, dtype=torch.bfloat16)
        yd = torch.empty(m.T, m.H, device=dev)
        ws = torch.empty(gq.gq_matvec_id_workspace(m.E, m.T, m.k, m.H), dtype=torch.uint8, device=dev)

        def run():
            for c in cps:
                if split:
                    gq.gq_route_topk_plan(lg, m.k, ids, rw, ws, stream)
                    gq.gq_matvec_id_glu(m.t, c["gate"], c["up"], m.E, m.F, m.H, (m.T, m.k), x4, "silu", hb, ws,
                                        stream)
                else:
                    gq.gq_route_matvec_id_glu(m.t, c["gate"], c["up"], m.E, m.F, m.H, lg, m.k, ids, rw, x4, "silu",
                                              hb, ws, stream)
                gq.gq_matvec_id(m.t, c["down"], m.E, m.H, m.F, (m.T, m.k), hb, True, yd, ws, rw, stream)

        return float(np.median(Timer(torch, run, stream).replays(2 * MIN_REPS))) / len(cps)
    if workload.startswith("prefill"):
        # "prefill" is the Q4_K product; "prefill:q6_k" / "prefill:q4_0" the others
        fmt = workload.split(":")[1] if ":" in workload else PREFILL.t
        L = next(m for m in WL.TIMED_MATMUL if m.t == fmt)
        W5, X5 = t_(L.weight()), t_(L.x_bf16_bits().view(np.int16)).view(torch.bfloat16)
        Y5 = torch.empty(L.M, L.N, device=dev)
        return float(np.median(Timer(torch, lambda: gq.gq_matmul(L.t, W5, L.N, L.K, X5, Y5, stream),
                                     stream).replays(30, warm=60)))
    raise SystemExit("unknown workload %r (headline, moe, moe:64, moe:split, prefill, prefill:q6_k, prefill:q4_0)"
                     % workload)


def abba(lib_a: str, lib_b: str, rounds: int, workload: str):
    """Compare two builds of libgq.so on one workload: `rounds` blocks of
    A, B, B, A, each run a fresh process (bench.py --measure-only with
    GQ_LIBGQ naming the build).  Reports the time ratio B / A with a 95%
    confidence interval over the blocks and the noise floor, the largest
    relative difference between two runs of the same build; a change is only
    called faster or slower when the interval excludes 1 and the ratio is
    further from 1 than that floor."""
    import subprocess
    libs = {"A": os.path.abspath(lib_a), "B": os.path.abspath(lib_b)}
    runs = {"A": [], "B": []}
    blocks = []
    for r in range(rounds):
        blk = {"A": [], "B": []}
        for which in "ABBA":
            env = dict(os.environ, GQ_LIBGQ=libs[which])
            out = subprocess.run([sys.executable, os.path.abspath(__file__), "--measure-only", "--workload", workload],
                                 env=env, capture_output=True, text=True, timeout=600)
            if out.returncode != 0:
                raise SystemExit("run %s failed:\n%s" % (which, out.stderr[-2000:]))
            ms = json.loads(out.stdout.strip().splitlines()[-1])["ms_per_step"]
            runs[which].append(ms)
            blk[which].append(ms)
            print("block %d %s: %.5f ms" % (r, which, ms), file=sys.stderr, flush=True)
        blocks.append(sum(blk["B"]) / sum(blk["A"]))
    ratio = sum(runs["B"]) / sum(runs["A"])
    n = len(blocks)
    mean = sum(blocks) / n
    sd = (sum((b - mean) ** 2 for b in blocks) / (n - 1)) ** 0.5 if n > 1 else float("nan")
    t975 = {1: 12.706, 2: 4.303, 3: 3.182, 4: 2.776, 5: 2.571, 6: 2.447, 7: 2.365, 8: 2.306, 9: 2.262}.get(n - 1, 2.0)
    half = t975 * sd / n ** 0.5
    noise = max((max(v) - min(v)) / (sum(v) / len(v)) for v in runs.values())
    if mean + half < 1 and 1 - ratio > noise:
        verdict = "B faster"
    elif mean - half > 1 and ratio - 1 > noise:
        verdict = "B slower"
    else:
        verdict = "no difference beyond the noise"
    print(json.dumps({"workload": workload, "lib_a": libs["A"], "lib_b": libs["B"], "blocks": n,
                      "ms_a": runs["A"], "ms_b": runs["B"], "ratio_b_over_a": round(ratio, 4),
                      "ci95": [round(mean - half, 4), round(mean + half, 4)], "noise_floor": round(noise, 4),
                      "verdict": verdict}))


def cpu_info() -> tuple[str, int, int]:
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, os.cpu_count() or 1, usable


def cpu_baseline(launches, host, xs):
    """The oracle (plain C: fp32 dequant, fp64 dot) over the headline layer on
    the host: once on one thread, once with one thread per usable core (at
    most 16, the host share of one GPU) over row ranges of each projection
    (ctypes releases the interpreter lock during the call)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as orc
    model, nproc, usable = cpu_info()
    threads = max(1, min(16, usable))
    xh = {L.name: xs[L.name].cpu().numpy() for L in launches}
    nbytes = sum(host[L.name].nbytes for L in launches)

    def layer(pool, parts):
        futs = []
        for L in launches:
            step = -(-L.N // parts)
            for r0 in range(0, L.N, step):
                futs.append(pool.submit(orc.matvec, L.t, host[L.name], L.N, L.K, xh[L.name],
                                        (r0, min(L.N, r0 + step))))
        for f in futs:
            f.result()

    res = {}
    for n in (1, threads):
        with ThreadPoolExecutor(n) as pool:
            tc = time.perf_counter()
            nrep = 0
            while True:
                layer(pool, n)
                nrep += 1
                if time.perf_counter() - tc > 8.0 or nrep >= 200:
                    break
            res[n] = ((time.perf_counter() - tc) / nrep, nrep)
    dt, nrep = res[threads]
    dt1, nrep1 = res[1]
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the whole 7-projection Q4_K layer at batch 1 (%d packed bytes) as the four launches' row "
                      "ranges split over %d threads, %d repetition(s), %.4f s per layer (plain C: fp32 dequant + "
                      "fp64 dot)" % (nbytes, threads, nrep, dt),
            "single_thread": {"value": round(nbytes / dt1 / 1e9, 4), "s_per_layer": round(dt1, 4),
                              "repetitions": nrep1},
            "host": {"cpu_model": model, "nproc": nproc, "usable_cores": usable}}


def bench_context(torch, gq, dev, stream, t_):
    """The other workloads, each timed the same way (graph of back-to-back
    launches over rotated copies), built from the same launch lists the
    parity tests check."""
    res = {}

    def x_dev(L):
        x = L.x()
        if L.xdt == "bf16":
            from block_quantized_weight_q4_amd import synth
            return t_(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16)
        return t_(x)

    def time_launches(group, reps):
        """Mean us per pass of `group` (launches in order) over rotated copies."""
        host = {L.name: L.weight() for L in group}
        nb = sum(w.nbytes for w in host.values())
        cps = [{k: t_(v) for k, v in host.items()} for _ in range(n_copies(nb))]
        xs = {L.name: x_dev(L) for L in group}
        ys = {L.name: torch.empty(L.batch, L.N, device=dev) for L in group}

        def run():
            for c in cps:
                for L in group:
                    gq.gq_matvec(L.t, c[L.name], L.N, L.K, xs[L.name], ys[L.name], stream)

        ms = float(np.median(Timer(torch, run, stream).replays(reps))) / len(cps)
        del cps
        torch.cuda.empty_cache()
        return ms * 1e3, nb

    by_wl = {}
    for L in WL.TIMED_MATVEC:
        by_wl.setdefault((L.workload, L.batch), []).append(L)
    for (wl, B), group in by_wl.items():
        if group == WL.HEADLINE:
            continue  # the headline
        us, nb = time_launches(group, MIN_REPS)
        entry = {"launches": ", ".join("%s %dx%d" % (L.name, L.N, L.K) if L.name != "w" else "%dx%d" % (L.N, L.K)
                                       for L in group),
                 "us": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1)}
        if len(group) > 1:
            entry["tokens_per_s_equiv"] = round(B / (us * 1e-6), 1)
        name = wl if wl.endswith("_b%d" % B) else "%s_b%d" % (wl, B)
        res["%s_%s" % (name, group[0].xdt)] = entry

    # dense layer at batch 1 with the fused gated unit: qkv, o, then
    # h = silu(gate x) * (up x) in one launch feeding the down projection
    G = WL.TIMED_GLU[0]
    qkv, o, _, down = WL.HEADLINE
    wq, wo, wd = qkv.weight(), o.weight(), down.weight()
    wg, wu = G.weights()
    lb = WL.layer_bytes("dense")
    cpf = [{"qkv": t_(wq), "o": t_(wo), "gate": t_(wg), "up": t_(wu), "down": t_(wd)} for _ in range(n_copies(lb))]
    xq, xo, xf = t_(qkv.x()), t_(o.x()), t_(G.x())
    yq, yo = torch.empty(1, qkv.N, device=dev), torch.empty(1, o.N, device=dev)
    hf, yd = torch.empty(1, G.N, device=dev), torch.empty(1, down.N, device=dev)

    def pf():
        for c in cpf:
            gq.gq_matvec("q4_k", c["qkv"], qkv.N, qkv.K, xq, yq, stream)
            gq.gq_matvec("q4_k", c["o"], o.N, o.K, xo, yo, stream)
            gq.gq_matvec_glu(G.t, c["gate"], c["up"], G.N, G.K, xf, G.act, hf, stream)
            gq.gq_matvec("q4_k", c["down"], down.N, down.K, hf, yd, stream)

    ms = float(np.median(Timer(torch, pf, stream).replays(MIN_REPS))) / len(cpf)
    res["dense_b1_fused_glu_f32"] = {"launches": "qkv, o, silu(gate)*up, down(h)", "us": round(ms * 1e3, 2),
                                     "GBps": round(lb / (ms * 1e-3) / 1e9, 1)}
    del cpf
    torch.cuda.empty_cache()

    # routed experts
    m = WL.MOE
    lg_t = t_(m.logits())
    ids_t = torch.empty((m.T, m.k), dtype=torch.int32, device=dev)
    rw_t = torch.empty((m.T, m.k), device=dev)
    gq.gq_route_topk(lg_t, m.k, ids_t, rw_t, stream)
    stream.synchronize()
    distinct = len(np.unique(ids_t.cpu().numpy()))
    ex = m.experts()
    layer_all = sum(v.nbytes for v in ex.values())
    read_bytes = layer_all // m.E * distinct
    cp4 = [{kk: t_(v) for kk, v in ex.items()} for _ in range(n_copies(layer_all))]
    x4 = t_(m.x())
    h4 = t_(m.h())
    yg = torch.empty(m.T, m.k, m.F, device=dev)
    yu = torch.empty(m.T, m.k, m.F, device=dev)
    yd = torch.empty(m.T, m.H, device=dev)
    wsz = max(gq.gq_matvec_id_workspace(m.E, m.T, m.k, m.F), gq.gq_matvec_id_workspace(m.E, m.T, m.k, m.H))
    ws = [torch.empty(wsz, dtype=torch.uint8, device=dev) for _ in range(3)]

    def p4():
        for c in cp4:
            gq.gq_route_topk(lg_t, m.k, ids_t, rw_t, stream)
            gq.gq_matvec_id(m.t, c["gate"], m.E, m.F, m.H, ids_t, x4, False, yg, ws[0], None, stream)
            gq.gq_matvec_id(m.t, c["up"], m.E, m.F, m.H, ids_t, x4, False, yu, ws[1], None, stream)
            gq.gq_matvec_id(m.t, c["down"], m.E, m.H, m.F, ids_t, h4, True, yd, ws[2], rw_t, stream)

    ms = float(np.median(Timer(torch, p4, stream).replays(MIN_REPS))) / len(cp4)
    res["moe_q4_0_128x_h2816_f704_t8_top8"] = {
        "launches": "route_topk, gate, up, down (weighted)",
        "us_per_layer": round(ms * 1e3, 2), "distinct_experts": distinct, "packed_bytes_read": read_bytes,
        "GBps": round(read_bytes / (ms * 1e-3) / 1e9, 1),
        "tokens_per_s_equiv_30_layers": round(m.T / (30 * ms * 1e-3), 1)}

    # the same layer with the routed gated unit in one launch; h (bf16) feeds
    # the down projection directly
    hb = torch.empty((m.T, m.k, m.F), device=dev, dtype=torch.bfloat16)

    def p5():
        for c in cp4:
            # routing and the group table in one launch; both products use the table
            gq.gq_route_topk_plan(lg_t, m.k, ids_t, rw_t, ws[0], stream)
            gq.gq_matvec_id_glu(m.t, c["gate"], c["up"], m.E, m.F, m.H, (m.T, m.k), x4, "silu", hb, ws[0], stream)
            gq.gq_matvec_id(m.t, c["down"], m.E, m.H, m.F, (m.T, m.k), hb, True, yd, ws[0], rw_t, stream)

    ms = float(np.median(Timer(torch, p5, stream).replays(MIN_REPS))) / len(cp4)
    res["moe_q4_0_128x_h2816_f704_t8_top8_fused_glu"] = {
        "launches": "route_topk + group table, gate|up + SiLU (bf16 h), down (weighted), both on that table",
        "us_per_layer": round(ms * 1e3, 2), "distinct_experts": distinct, "packed_bytes_read": read_bytes,
        "GBps": round(read_bytes / (ms * 1e-3) / 1e9, 1),
        "tokens_per_s_equiv_30_layers": round(m.T / (30 * ms * 1e-3), 1)}

    # the routing inside the gated unit's launch (every workgroup routes the
    # 8 tokens itself): three launches per layer
    def p6():
        for c in cp4:
            gq.gq_route_matvec_id_glu(m.t, c["gate"], c["up"], m.E, m.F, m.H, lg_t, m.k, ids_t, rw_t, x4, "silu",
                                      hb, ws[0], stream)
            gq.gq_matvec_id(m.t, c["down"], m.E, m.H, m.F, (m.T, m.k), hb, True, yd, ws[0], rw_t, stream)

    ms = float(np.median(Timer(torch, p6, stream).replays(MIN_REPS))) / len(cp4)
    res["moe_q4_0_128x_h2816_f704_t8_top8_fused_routed_glu"] = {
        "launches": "route_topk inside gate|up + SiLU (bf16 h), down (weighted) on the table it leaves",
        "us_per_layer": round(ms * 1e3, 2), "distinct_experts": distinct, "packed_bytes_read": read_bytes,
        "GBps": round(read_bytes / (ms * 1e-3) / 1e9, 1),
        "tokens_per_s_equiv_30_layers": round(m.T / (30 * ms * 1e-3), 1)}
    del cp4
    torch.cuda.empty_cache()
    # the same fused layer for a 64-token block (groups of up to 8 slots:
    # about 127 groups over 125 distinct experts)
    m64 = WL.MoeLayer(T=64)
    ms64 = measure(torch, gq, dev, stream, t_, "moe:64")
    res["moe_q4_0_128x_h2816_f704_t64_top8_fused_glu"] = {
        "launches": "as the 8-token fused layer", "us_per_layer": round(ms64 * 1e3, 2),
        "tokens_per_s_equiv_30_layers": round(m64.T / (30 * ms64 * 1e-3), 1)}
    return res


if __name__ == "__main__":
    main()
