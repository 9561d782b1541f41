"""Benchmark of the packed-weight decode product on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decoder layer of Q4_K products at batch 1, hidden 2560:
q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up 9728x2560, down 2560x9728
(56,770,560 packed bytes).  q|k|v and gate|up read the same activation vector
and are issued as one launch each over their row-concatenated weights (rows
back to back, as a model loader stores them), so a step is four launches:
qkv, o, gate|up, down.  Weights rotate over >= 1 GiB of distinct copies so every
step reads HBM, not the 256 MB last-level cache.  Inputs are resident in HBM
before the timed region.

Printed: one JSON line with the whole-step packed-weight rate (value, GB/s),
the dominant kernel's roofline figures (gate|up, timed per launch with HIP
events on the launch stream) and the CPU oracle timed on the host for the same
layer.  Extra keys report the unfused seven-launch layer, and every other
workload shape as context.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "packed-weight GB/s (% of HBM peak), Q4_K GEMV batch 1; prefill TFLOP/s"
ROTATE_BYTES = 1 << 30

DENSE = [("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560), ("o", 2560, 4096),
         ("gate", 9728, 2560), ("up", 9728, 2560), ("down", 2560, 9728)]


def row_bytes(K: int) -> int:
    return K // 256 * 144


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the context workloads")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the product is sharded by output rows across GPUs in a larger deployment; "
              "see DESIGN.md).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_quantized_weight_q4_amd as gq
    from block_quantized_weight_q4_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---- weights: one seeded layer, copied to >= 1 GiB of distinct buffers
    g = synth.rng(0x67510002, 0)
    mats = {name: synth.weight("q4_k", synth.rng(0x67510002, i), N, K) for i, (name, N, K) in enumerate(DENSE)}
    qkv = np.concatenate([mats["q"], mats["k"], mats["v"]], axis=0)
    gu = np.concatenate([mats["gate"], mats["up"]], axis=0)
    layer_bytes = sum(m.nbytes for m in mats.values())
    n_copies = max(2, -(-ROTATE_BYTES // layer_bytes))
    host = {"qkv": qkv, "o": mats["o"], "gu": gu, "down": mats["down"]}
    copies = []
    for c in range(n_copies):
        copies.append({k: torch.from_numpy(v).to(dev) for k, v in host.items()})
    # activations (distinct vectors per launch; resident before timing)
    xs = {
        "qkv": torch.from_numpy(synth.normal_f32(g, (1, 2560))).to(dev),
        "o": torch.from_numpy(synth.normal_f32(g, (1, 4096))).to(dev),
        "gu": torch.from_numpy(synth.normal_f32(g, (1, 2560))).to(dev),
        "down": torch.from_numpy(synth.normal_f32(g, (1, 9728))).to(dev),
    }
    shapes = {"qkv": (6144, 2560), "o": (2560, 4096), "gu": (19456, 2560), "down": (2560, 9728)}
    ys = {k: torch.empty(1, n, device=dev) for k, (n, _) in shapes.items()}

    def step(c):
        w = copies[c % n_copies]
        for k in ("qkv", "o", "gu", "down"):
            n, kk = shapes[k]
            gq.gq_matvec("q4_k", w[k], n, kk, xs[k], ys[k], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    value = layer_bytes / (ms_step * 1e-3) / 1e9

    # ---- dominant kernel: gate|up, per-launch HIP events on the launch stream
    gu_bytes = gu.nbytes
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.warmup):
        gq.gq_matvec("q4_k", copies[i % n_copies]["gu"], 19456, 2560, xs["gu"], ys["gu"], stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        a, b = ev[i]
        a.record(stream)
        gq.gq_matvec("q4_k", copies[i % n_copies]["gu"], 19456, 2560, xs["gu"], ys["gu"], stream)
        b.record(stream)
    torch.cuda.synchronize()
    gu_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9

    # ---- unfused seven-launch layer (context)
    sep = {name: [torch.from_numpy(m).to(dev) for _ in range(max(2, -(-ROTATE_BYTES // layer_bytes)))]
           for name, m in mats.items()} if not args.quick else None
    unfused = None
    if sep is not None:
        xk = {2560: xs["qkv"], 4096: xs["o"], 9728: xs["down"]}
        yk = {name: torch.empty(1, N, device=dev) for name, N, K in DENSE}
        nc = len(sep["q"])

        def step7(c):
            for name, N, K in DENSE:
                gq.gq_matvec("q4_k", sep[name][c % nc], N, K, xk[K], yk[name], stream)

        for i in range(args.warmup):
            step7(i)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            step7(i)
        t1.record(stream)
        torch.cuda.synchronize()
        ms7 = t0.elapsed_time(t1) / args.steps
        unfused = {"ms_per_layer": ms7, "GBps": layer_bytes / (ms7 * 1e-3) / 1e9, "launches": 7}
        del sep
    del copies
    torch.cuda.empty_cache()

    # ---- CPU oracle on the host (the same layer, single thread)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        xh = {2560: xs["qkv"].cpu().numpy(), 4096: xs["o"].cpu().numpy(), 9728: xs["down"].cpu().numpy()}
        tc = time.perf_counter()
        reps = 0
        while True:
            for name, N, K in DENSE:
                orc.matvec("q4_k", mats[name], N, K, xh[K])
            reps += 1
            if time.perf_counter() - tc > 10.0 or reps >= 20:
                break
        dt = (time.perf_counter() - tc) / reps
        cpu = {"value": layer_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "the full 7-projection Q4_K layer at batch 1, %d repetition(s), single thread "
                         "(plain C, fp32 dequant + fp64 dot), %.3f s per layer" % (reps, dt)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
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
            "launches_per_step": "qkv (6144x2560), o, gate|up (19456x2560), down",
            "batch": 1,
            "packed_bytes_per_step": layer_bytes,
            "weight_copies_rotated": n_copies,
            "activations": "fp32 N(0,1)",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_matvec Q4_K gate|up 19456x2560 batch 1",
                     "bytes_per_launch": gu_bytes, "avg_launch_ms": round(gu_ms, 5)},
        "cpu_baseline": cpu,
        "unfused_layer": unfused,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
