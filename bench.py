"""Benchmark of the packed-weight products on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu-baseline]
    python bench.py --pmc-pass            (the dominant kernel + a copy kernel, for rocprofv3 --pmc)
    python bench.py --traffic-summary FETCH_DIR WRITE_DIR   (writes profiles/<kernel>_traffic.txt)
    python bench.py --stats-summary DIR OUT.txt             (rocprofv3 --stats CSV -> text summary)

The step (the headline workload) is one decoder layer of Q4_K products at
batch 1, hidden 2560: q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up
9728x2560, down 2560x9728 -- 56,770,560 packed bytes.  q|k|v and gate|up read
the same activation vector and are issued as one launch each over their
row-concatenated weights (a loader stores them that way), so a step is four
dependent launches: qkv, o, gate|up, down.  Weights rotate over >= 1 GiB of
distinct copies so each step streams from HBM, not from the 256 MB last-level
cache; inputs are resident in HBM before the timed region.  The steps are
captured once in a HIP graph that walks every copy; the timed region replays
it, bracketed by device synchronisation and HIP events on the launch stream.

One JSON line: value = packed-weight GB/s of the whole step; roofline = the
dominant kernel (gate|up, 28,016,640 B per launch) timed over back-to-back
launches of it alone; cpu_baseline = the CPU oracle on the same layer; plus
the prefill product's TFLOP/s and the other workloads as context.

roofline.traffic is the HBM bytes per launch of that kernel from two
rocprofv3 --pmc runs of `--pmc-pass` (FETCH_SIZE, then WRITE_SIZE), each
scaled by the factor that makes the same counter read right for a plain copy
kernel of known size.  The summary file records a hash of the kernel's
sources; when the sources have changed since, traffic is reported as null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "packed-weight GB/s (% of HBM peak), Q4_K GEMV batch 1; prefill TFLOP/s"
ROTATE_BYTES = 1 << 30

DENSE = [("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560), ("o", 2560, 4096),
         ("gate", 9728, 2560), ("up", 9728, 2560), ("down", 2560, 9728)]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline only (no context workloads)")
    ap.add_argument("--context-only", action="store_true",
                    help="only the context workloads (one JSON line of them; for kernel traces)")
    ap.add_argument("--pmc-pass", action="store_true", help="run the dominant kernel 8x and one copy kernel")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--stats-summary", nargs=2, metavar=("DIR", "OUT"))
    return ap.parse_args()


# ------------------------------------------------------------ traffic
GU_N, GU_K = 19456, 2560
GU_KERNEL = "k_matvec<2, 0, 1"          # Q4_K, fp32 activations, batch 1
COPY_BYTES = 64 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "matvec_q4k_gateup_19456x2560_b1_traffic.txt")
KERNEL_SOURCES = ["gq_device.h", "gq_gemv_core.h", "gq_matvec.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_quantized_weight_q4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_pass():
    """The dominant kernel (gate|up, batch 1) over 8 distinct weight copies,
    then torch's elementwise add over a 64 MiB fp32 tensor: 64 MiB read,
    64 MiB written, the calibration for the byte counters."""
    import torch
    import block_quantized_weight_q4_amd as gq
    from block_quantized_weight_q4_amd import synth
    dev = torch.device("cuda:0")
    W = synth.weight("q4_k", synth.rng(0x67510002, 4), GU_N, GU_K)
    Ws = [torch.from_numpy(W).to(dev) for _ in range(8)]
    x = torch.from_numpy(synth.normal_f32(synth.rng(0x67510002, 100), (1, GU_K))).to(dev)
    y = torch.empty(1, GU_N, device=dev)
    for w in Ws:
        gq.gq_matvec("q4_k", w, GU_N, GU_K, x, y)
    torch.cuda.synchronize()
    src = torch.empty(COPY_BYTES // 4, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    print("pmc pass done", flush=True)


def _counter_means(d: str) -> dict:
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
    algo = GU_N * (GU_K // 256) * 144
    text = ["# HBM traffic of the Q4_K gate|up product (19456 x 2560, batch 1, fp32 x)",
            "",
            "kernel: %s (Q4_K, fp32 activations, batch 1)" % kname.split("(unsigned")[0].replace("void ", ""),
            "source_sha256: %s" % kernel_source_hash(),
            "commands (from the repository root, on the GPU host):",
            "  timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -- python3 bench.py --pmc-pass",
            "  timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -- python3 bench.py --pmc-pass",
            "  python bench.py --traffic-summary <FETCH_DIR> <WRITE_DIR>",
            ""] + out_lines + [
            "",
            "traffic_bytes_per_launch: %.0f" % traffic,
            "algorithmic_bytes_per_launch: %d (packed weights) + %d (x) + %d (y)" % (algo, GU_K * 4, GU_N * 4),
            "traffic / algorithmic: %.4f" % (traffic / (algo + GU_K * 4 + GU_N * 4))]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def read_traffic():
    """traffic_bytes_per_launch from the committed summary, or None when the
    kernel sources changed since it was taken (or there is none)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"source_sha256: (\w+)", text)
    t = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


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
        k = (r["Kernel_Name"][:80], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        per.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "per launch shape (grid = work-items):",
              "%-80s %9s %5s %7s %10s %10s" % ("kernel", "grid", "wg", "calls", "avg_us", "median_us")]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        lines.append("%-80s %9d %5d %7d %10.3f %10.3f" % (k[0], k[1], k[2], len(v), sum(v) / len(v), v[len(v) // 2]))
    with open(out, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


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

    def time(self, reps: int, warm: int = 2) -> float:
        """Mean ms per replay over `reps` replays."""
        torch = self.torch
        for _ in range(warm):
            self.graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for _ in range(reps):
            self.graph.replay()
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps


def main():
    args = parse()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    if args.stats_summary:
        return stats_summary(*args.stats_summary)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the products shard by "
              "output rows across GPUs).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.pmc_pass:
        return pmc_pass()

    import torch
    import block_quantized_weight_q4_amd as gq
    from block_quantized_weight_q4_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    side = torch.cuda.Stream()  # graphs are captured on a non-default stream
    torch.cuda.set_stream(side)
    stream = torch.cuda.current_stream()

    def t_(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if args.context_only:
        print(json.dumps({"context": bench_context(torch, gq, synth, dev, stream, t_)}), flush=True)
        return

    # ------------------------------------------------ headline: dense layer
    mats = {name: synth.weight("q4_k", synth.rng(0x67510002, i), N, K) for i, (name, N, K) in enumerate(DENSE)}
    host = {"qkv": np.concatenate([mats["q"], mats["k"], mats["v"]]), "o": mats["o"],
            "gu": np.concatenate([mats["gate"], mats["up"]]), "down": mats["down"]}
    shapes = {"qkv": (6144, 2560), "o": (2560, 4096), "gu": (19456, 2560), "down": (2560, 9728)}
    layer_bytes = sum(m.nbytes for m in mats.values())
    n_copies = max(2, -(-ROTATE_BYTES // layer_bytes))
    copies = [{k: t_(v) for k, v in host.items()} for _ in range(n_copies)]
    g = synth.rng(0x67510002, 100)
    xs = {k: t_(synth.normal_f32(g, (1, K))) for k, (N, K) in shapes.items()}
    ys = {k: torch.empty(1, N, device=dev) for k, (N, K) in shapes.items()}

    def layer_pass():
        for c in copies:
            for k in ("qkv", "o", "gu", "down"):
                n, kk = shapes[k]
                gq.gq_matvec("q4_k", c[k], n, kk, xs[k], ys[k], stream)

    tl = Timer(torch, layer_pass, stream)
    reps = max(1, args.steps // n_copies)
    tl.time(max(1, args.warmup // n_copies))
    ms_pass = tl.time(reps)
    steps = reps * n_copies
    ms_step = ms_pass / n_copies
    value = layer_bytes / (ms_step * 1e-3) / 1e9

    # dominant kernel: gate|up alone, back to back over the copies
    def gu_pass():
        for c in copies:
            gq.gq_matvec("q4_k", c["gu"], 19456, 2560, xs["gu"], ys["gu"], stream)

    tg = Timer(torch, gu_pass, stream)
    gu_ms = tg.time(max(2, reps)) / n_copies
    gu_bytes = host["gu"].nbytes
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    del tl, tg, copies
    torch.cuda.empty_cache()

    context = {}
    # ------------------------------------------------ prefill product
    M, N5, K5 = 3015, 17408, 5120
    W5 = t_(synth.weight("q4_k", synth.rng(0x67510005, 0), N5, K5))
    X5 = t_(synth.bf16_bits(synth.normal_f32(synth.rng(0x67510005, 1), (M, K5))).view(np.int16)).view(torch.bfloat16)
    Y5 = torch.empty(M, N5, device=dev)
    tp = Timer(torch, lambda: gq.gq_matmul("q4_k", W5, N5, K5, X5, Y5, stream), stream)
    # the matrix cores reach their sustained clock only after some tens of
    # milliseconds of this load: replay well past that before timing
    ms_mm = tp.time(30, warm=60)
    flops = 2.0 * M * N5 * K5
    prefill = {"workload": "q4_k_prefill_3015x17408x5120_bf16", "ms": round(ms_mm, 4),
               "TFLOPs": round(flops / (ms_mm * 1e-3) / 1e12, 2),
               "frac_bf16_dense_peak": round(flops / (ms_mm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
               "tokens_per_s": round(M / (ms_mm * 1e-3), 1)}
    del tp, W5, X5, Y5
    torch.cuda.empty_cache()
    # the same prefill length through the other formats of a Q4_K_M layer:
    # the Q6_K down projection (5120 x 17408) and a Q4_0 matrix of the c5 shape
    others = {}
    for t5, N6, K6 in (("q6_k", 5120, 17408), ("q4_0", 17408, 5120)):
        W6 = t_(synth.weight(t5, synth.rng(0x67510005, 2), N6, K6))
        X6 = t_(synth.bf16_bits(synth.normal_f32(synth.rng(0x67510005, 3), (M, K6))).view(np.int16)).view(
            torch.bfloat16)
        Y6 = torch.empty(M, N6, device=dev)
        tp = Timer(torch, lambda: gq.gq_matmul(t5, W6, N6, K6, X6, Y6, stream), stream)
        ms6 = tp.time(20, warm=40)
        others["%s_prefill_%dx%dx%d_bf16" % (t5, M, N6, K6)] = {
            "ms": round(ms6, 4), "TFLOPs": round(2.0 * M * N6 * K6 / (ms6 * 1e-3) / 1e12, 2)}
        del tp, W6, X6, Y6
        torch.cuda.empty_cache()
    prefill["other_formats"] = others

    if not args.quick:
        context = bench_context(torch, gq, synth, dev, stream, t_)

    # ------------------------------------------------ CPU oracle on the host
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        xh = {2560: xs["qkv"].cpu().numpy(), 4096: xs["o"].cpu().numpy(), 9728: xs["down"].cpu().numpy()}
        tc = time.perf_counter()
        nrep = 0
        while True:
            for name, N, K in DENSE:
                orc.matvec("q4_k", mats[name], N, K, xh[K])
            nrep += 1
            if time.perf_counter() - tc > 10.0 or nrep >= 30:
                break
        dt = (time.perf_counter() - tc) / nrep
        cpu = {"value": round(layer_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "the whole 7-projection Q4_K layer at batch 1 (56,770,560 packed bytes), %d "
                         "repetition(s) on one host thread (plain C: fp32 dequant + fp64 dot), %.3f s per layer"
                         % (nrep, dt)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
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
            "weight_copies_rotated": n_copies,
            "activations": "fp32 N(0,1)",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s_equiv": round(value / 2.74, 1),
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
                     "kernel": "k_matvec<Q4_K, fp32, batch 1> gate|up 19456x2560",
                     "bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_ms * 1e3, 3)},
        "cpu_baseline": cpu,
        "prefill": prefill,
        "context": context,
    }
    print(json.dumps(out))


def bench_context(torch, gq, synth, dev, stream, t_):
    """The other workloads, each timed the same way (graph of back-to-back
    launches over rotated copies)."""
    res = {}

    def rotated(make, nbytes):
        return [make() for _ in range(max(2, -(-ROTATE_BYTES // nbytes)))]

    # Q4_0 2048x2048, batch 1
    w1 = synth.weight("q4_0", synth.rng(0x67510001, 0), 2048, 2048)
    c1 = [t_(w1) for _ in range(max(2, -(-(256 << 20) // w1.nbytes)))]
    x1 = t_(synth.normal_f32(synth.rng(0x67510001, 1), (1, 2048)))
    y1 = torch.empty(1, 2048, device=dev)

    def p1():
        for c in c1:
            gq.gq_matvec("q4_0", c, 2048, 2048, x1, y1, stream)

    ms = Timer(torch, p1, stream).time(20) / len(c1)
    res["q4_0_2048x2048_b1"] = {"us": round(ms * 1e3, 3), "GBps": round(w1.nbytes / (ms * 1e-3) / 1e9, 1)}
    del c1

    # Q5_K (the Q5_K_M variant's main type) at the hidden-5120 gate shape, batch 1 and 8, bf16
    w5 = synth.weight("q5_k", synth.rng(0x67510007, 0), 17408, 5120)
    c5 = [t_(w5) for _ in range(max(2, -(-ROTATE_BYTES // w5.nbytes)))]
    for B in (1, 8):
        x5 = t_(synth.bf16_bits(synth.normal_f32(synth.rng(0x67510007, B), (B, 5120))).view(np.int16)).view(
            torch.bfloat16)
        y5 = torch.empty(B, 17408, device=dev)

        def p5():
            for c in c5:
                gq.gq_matvec("q5_k", c, 17408, 5120, x5, y5, stream)

        ms = Timer(torch, p5, stream).time(10) / len(c5)
        res["q5_k_17408x5120_bf16_b%d" % B] = {"us": round(ms * 1e3, 3),
                                               "GBps": round(w5.nbytes / (ms * 1e-3) / 1e9, 1)}
    del c5
    torch.cuda.empty_cache()

    # dense layer at batch 1 with the fused gated unit: qkv, o, then
    # h = silu(gate x) * (up x) in one launch feeding the down projection
    mats = {name: synth.weight("q4_k", synth.rng(0x67510002, i), N, K) for i, (name, N, K) in enumerate(DENSE)}
    lb = sum(m.nbytes for m in mats.values())
    qkv = np.concatenate([mats["q"], mats["k"], mats["v"]])
    cpf = [{"qkv": t_(qkv), "o": t_(mats["o"]), "gate": t_(mats["gate"]), "up": t_(mats["up"]),
            "down": t_(mats["down"])} for _ in range(max(2, -(-ROTATE_BYTES // lb)))]
    gx = synth.rng(0x67510002, 100)
    xq = t_(synth.normal_f32(gx, (1, 2560)))
    xo = t_(synth.normal_f32(gx, (1, 4096)))
    xf = t_(synth.normal_f32(gx, (1, 2560)))
    yq, yo = torch.empty(1, 6144, device=dev), torch.empty(1, 2560, device=dev)
    hf, yd = torch.empty(1, 9728, device=dev), torch.empty(1, 2560, device=dev)

    def pf():
        for c in cpf:
            gq.gq_matvec("q4_k", c["qkv"], 6144, 2560, xq, yq, stream)
            gq.gq_matvec("q4_k", c["o"], 2560, 4096, xo, yo, stream)
            gq.gq_matvec_glu("q4_k", c["gate"], c["up"], 9728, 2560, xf, "silu", hf, stream)
            gq.gq_matvec("q4_k", c["down"], 2560, 9728, hf, yd, stream)

    ms = Timer(torch, pf, stream).time(20) / len(cpf)
    res["q4_k_dense_layer_b1_fused_glu"] = {
        "launches": "qkv, o, silu(gate)*up, down(h)", "us_per_layer": round(ms * 1e3, 2),
        "GBps": round(lb / (ms * 1e-3) / 1e9, 1)}
    del cpf
    torch.cuda.empty_cache()

    # dense layer at batch 4
    mats = {name: synth.weight("q4_k", synth.rng(0x67510002, i), N, K) for i, (name, N, K) in enumerate(DENSE)}
    host = {"qkv": (np.concatenate([mats["q"], mats["k"], mats["v"]]), 6144, 2560), "o": (mats["o"], 2560, 4096),
            "gu": (np.concatenate([mats["gate"], mats["up"]]), 19456, 2560), "down": (mats["down"], 2560, 9728)}
    lb = sum(m.nbytes for m in mats.values())
    cp = [{k: t_(v[0]) for k, v in host.items()} for _ in range(max(2, -(-ROTATE_BYTES // lb)))]
    x4 = {k: t_(synth.normal_f32(synth.rng(0x67510002, 200), (4, v[2]))) for k, v in host.items()}
    y4 = {k: torch.empty(4, v[1], device=dev) for k, v in host.items()}

    def p2():
        for c in cp:
            for k, v in host.items():
                gq.gq_matvec("q4_k", c[k], v[1], v[2], x4[k], y4[k], stream)

    ms = Timer(torch, p2, stream).time(5) / len(cp)
    res["q4_k_dense_layer_b4"] = {"us_per_layer": round(ms * 1e3, 2), "GBps": round(lb / (ms * 1e-3) / 1e9, 1),
                                  "tokens_per_s_equiv": round(4 * lb / (ms * 1e-3) / 1e9 / 2.74, 1)}
    del cp
    torch.cuda.empty_cache()

    # mixed Q4_K / Q6_K layer, hidden 5120, FFN 17408, bf16 activations
    specs = [("qk", "q4_k", [("q", 5120), ("k", 1024)], 5120), ("v", "q6_k", [("v", 1024)], 5120),
             ("o", "q4_k", [("o", 5120)], 5120), ("gu", "q4_k", [("gate", 17408), ("up", 17408)], 5120),
             ("down", "q6_k", [("down", 5120)], 17408)]
    idx = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}
    hw = {}
    lb3 = 0
    for name, t, parts, K in specs:
        arrs = [synth.weight(t, synth.rng(0x67510003, idx[p]), n, K) for p, n in parts]
        hw[name] = (np.concatenate(arrs), t, sum(n for _, n in parts), K)
        lb3 += sum(a.nbytes for a in arrs)
    cp3 = [{k: t_(v[0]) for k, v in hw.items()} for _ in range(max(2, -(-ROTATE_BYTES // lb3)))]
    for B in (1, 2, 8, 16):
        xb = {k: t_(synth.bf16_bits(synth.normal_f32(synth.rng(0x67510003, 300 + B), (B, v[3]))).view(np.int16))
              .view(torch.bfloat16) for k, v in hw.items()}
        yb = {k: torch.empty(B, v[2], device=dev) for k, v in hw.items()}

        def p3():
            for c in cp3:
                for k, v in hw.items():
                    gq.gq_matvec(v[1], c[k], v[2], v[3], xb[k], yb[k], stream)

        ms = Timer(torch, p3, stream).time(5) / len(cp3)
        res["mixed_layer_h5120_bf16_b%d" % B] = {"us_per_layer": round(ms * 1e3, 2),
                                                 "GBps": round(lb3 / (ms * 1e-3) / 1e9, 1),
                                                 "tokens_per_s_equiv": round(B / (ms * 1e-3), 1)}
    del cp3
    torch.cuda.empty_cache()

    # MoE routed experts: 128 experts, hidden 2816, FFN 704, 8 tokens top-8
    E, H, F, T, k = 128, 2816, 704, 8, 8
    g = synth.rng(0x67510004, 0)
    logits = synth.router_logits(g, T, E)
    lg_t = t_(logits)
    ids_t = torch.empty((T, k), dtype=torch.int32, device=dev)
    rw_t = torch.empty((T, k), device=dev)
    gq.gq_route_topk(lg_t, k, ids_t, rw_t, stream)
    stream.synchronize()
    distinct = len(np.unique(ids_t.cpu().numpy()))
    ex = {"gate": synth.weight("q4_0", synth.rng(0x67510004, 1), E * F, H),
          "up": synth.weight("q4_0", synth.rng(0x67510004, 2), E * F, H),
          "down": synth.weight("q4_0", synth.rng(0x67510004, 3), E * H, F)}
    layer_all = sum(v.nbytes for v in ex.values())
    read_bytes = layer_all // E * distinct
    cp4 = [{kk: t_(v) for kk, v in ex.items()} for _ in range(max(2, -(-ROTATE_BYTES // layer_all)))]
    x4 = t_(synth.normal_f32(g, (T, H)))
    h4 = t_(synth.normal_f32(g, (T, k, F)))
    yg = torch.empty(T, k, F, device=dev)
    yu = torch.empty(T, k, F, device=dev)
    yd = torch.empty(T, H, device=dev)
    wsz = max(gq.gq_matvec_id_workspace(E, T, k, F), gq.gq_matvec_id_workspace(E, T, k, H))
    ws = [torch.empty(wsz, dtype=torch.uint8, device=dev) for _ in range(3)]

    def p4():
        for c in cp4:
            gq.gq_route_topk(lg_t, k, ids_t, rw_t, stream)
            gq.gq_matvec_id("q4_0", c["gate"], E, F, H, ids_t, x4, False, yg, ws[0], None, stream)
            gq.gq_matvec_id("q4_0", c["up"], E, F, H, ids_t, x4, False, yu, ws[1], None, stream)
            gq.gq_matvec_id("q4_0", c["down"], E, H, F, ids_t, h4, True, yd, ws[2], rw_t, stream)

    ms = Timer(torch, p4, stream).time(10) / len(cp4)
    res["moe_q4_0_128x_h2816_f704_t8_top8"] = {
        "launches": "route_topk, gate, up, down (weighted); each routed call = group plan + product",
        "us_per_layer": round(ms * 1e3, 2), "distinct_experts": distinct, "packed_bytes_read": read_bytes,
        "GBps": round(read_bytes / (ms * 1e-3) / 1e9, 1),
        "tokens_per_s_equiv_30_layers": round(T / (30 * ms * 1e-3), 1)}

    # the same layer with the routed gated unit in one launch; h (bf16) feeds
    # the down projection directly
    hb = torch.empty((T, k, F), device=dev, dtype=torch.bfloat16)

    def p5():
        for c in cp4:
            gq.gq_route_topk(lg_t, k, ids_t, rw_t, stream)
            gq.gq_matvec_id_glu("q4_0", c["gate"], c["up"], E, F, H, ids_t, x4, "silu", hb, ws[0], stream)
            gq.gq_matvec_id("q4_0", c["down"], E, H, F, ids_t, hb, True, yd, ws[2], rw_t, stream)

    ms = Timer(torch, p5, stream).time(10) / len(cp4)
    res["moe_q4_0_128x_h2816_f704_t8_top8_fused_glu"] = {
        "launches": "route_topk, gate|up + SiLU (bf16 h), down (weighted); each routed call = group plan + product",
        "us_per_layer": round(ms * 1e3, 2), "distinct_experts": distinct, "packed_bytes_read": read_bytes,
        "GBps": round(read_bytes / (ms * 1e-3) / 1e9, 1),
        "tokens_per_s_equiv_30_layers": round(T / (30 * ms * 1e-3), 1)}
    del cp4
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
