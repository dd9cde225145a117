"""Benchmark of the attention hot path on one MI355X.

One step = one forward (fa_fwd) and one backward (fa_bwd's three stages:
delta preprocess, dK/dV, dQ) over the long-context workload: B=1, H=16,
N=16384, d=128, bf16, causal, scale 1/sqrt(128), Q/K/V/dO ~ N(0, 0.5) from the
seeded generator.  Inputs are resident in HBM before timing starts.

value = attention TFLOP/s of fwd+bwd = 3.5 * F_fwd / t_step with
F_fwd = 4 B H N^2 d / 2 (causal), i.e. backward counted as 2.5x forward.

Each stage is bracketed by HIP events recorded on the stream the library
launches on, so the per-kernel averages come from the timed steps themselves.
The roofline object describes the kernel with the largest average time.

cpu_baseline times the fp64 CPU oracle (forward + backward) on one head of the
same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s fwd+bwd (bf16, 1 GPU) and % of MFMA bf16 peak, N=1K–16K"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0


def flops_fwd(B, H, N, d, causal, cell_frac=1.0):
    f = 4.0 * B * H * N * N * d * cell_frac
    return f / 2 if causal else f


def kernel_flops(name, B, H, N, d, causal):
    """GEMM flops each kernel must execute per launch (visited score entries x 2d
    per product): fwd 2 products (S, PV), dkdv 4 (S, dP, dV, dK), dq 3 (S, dP, dQ)."""
    per_product = flops_fwd(B, H, N, d, causal) / 2
    return {"fwd": 2, "dkdv": 4, "dq": 3, "pre": 0}[name] * per_product


def run_gpu_bench(w, steps, warmup, inp):
    import numpy as np
    import torch

    import exact_io_aware_flashattention_amd as fa

    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(inp[n]).to(dev, torch.bfloat16) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    kw = dict(scale=w.scale, causal=w.causal)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, stream=stream, **kw)
        if ev:
            ev[1].record(stream)
        fa.fa_bwd_preprocess(o, do, delta, stream=stream)
        if ev:
            ev[2].record(stream)
        fa.fa_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, stream=stream, **kw)
        if ev:
            ev[3].record(stream)
        fa.fa_bwd_dq(q, k, v, do, lse, delta, dq, stream=stream, **kw)
        if ev:
            ev[4].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    names = ["fwd", "pre", "dkdv", "dq"]
    per = {n: 0.0 for n in names}
    for ev in evs:
        for j, n in enumerate(names):
            per[n] += ev[j].elapsed_time(ev[j + 1])
    per = {n: per[n] / steps for n in names}      # ms per launch
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(dq).all())
    return total_ms / steps, per, wall, (B, H, N, d)


COPY_BYTES = 256 << 20


def copy_calibration():
    """One device-to-device copy of COPY_BYTES: read COPY_BYTES, write COPY_BYTES.
    Its FETCH_SIZE / WRITE_SIZE readings scale the counters of the attention
    kernels to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def cpu_baseline(w, inp, heads=2):
    """fp64 oracle fwd + bwd on the first `heads` heads of the workload (all rows, all keys)."""
    import numpy as np

    from oracle import sparse
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    for h in range(heads):
        Q, K, V, dO = (inp[n][0, h].astype(np.float64) for n in ("q", "k", "v", "do"))
        sparse.head_forward(Q, K, V, w.scale, causal=w.causal)
        sparse.head_backward(Q, K, V, dO, w.scale, causal=w.causal)
    dt = time.perf_counter() - t0
    f = 3.5 * flops_fwd(1, heads, w.N, w.d, w.causal)
    return {"value": round(f / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"heads 0-{heads - 1} of {w.B * w.H} of the same workload (N={w.N}, d={w.d}, causal), "
                      f"fp64 forward+backward, {dt:.1f} s",
            "seconds": round(dt, 2)}


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "long_context_hbm_traffic.txt")
KERNEL_SYMBOL = {"fwd": "fwd_bf16_kernel<128, false>", "dkdv": "dkdv_bf16_kernel<128, false>",
                 "dq": "dq_bf16_kernel<128, false>", "pre": "bwd_pre_kernel"}


def kernel_source_hash():
    """SHA-256 over the HIP sources; counter readings are only reported while it matches."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_io_aware_flashattention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed counter summary, or {} when the
    kernels changed after the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return {}
    return {k[len("bytes_"):]: float(v) for k, v in kv.items() if k.startswith("bytes_")}


def summarize_counters(fetch_csv, write_csv, command):
    """Write the per-kernel HBM traffic summary from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch).  Each counter is scaled by its
    reading for the plain copy of COPY_BYTES made by --copy-calibration."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_name = next(n for n in fetch if "copyBuffer" in n)
    f_scale = (COPY_BYTES / 1024) / max(fetch[copy_name])
    w_scale = (COPY_BYTES / 1024) / max(write[copy_name])
    lines = ["# HBM traffic per launch, long-context workload (B=1 H=16 N=16384 d=128 bf16 causal)",
             f"# command: {command}",
             f"# calibration: a {COPY_BYTES >> 20} MiB device copy reads FETCH_SIZE {max(fetch[copy_name]):.1f} KiB "
             f"(scale {f_scale:.4f}) and WRITE_SIZE {max(write[copy_name]):.1f} KiB (scale {w_scale:.4f})",
             f"source_hash = {kernel_source_hash()}",
             f"fetch_scale = {f_scale:.6f}", f"write_scale = {w_scale:.6f}"]
    for key, sym in KERNEL_SYMBOL.items():
        fn = [n for n in fetch if sym in n or (key == "pre" and "bwd_pre" in n)]
        wn = [n for n in write if sym in n or (key == "pre" and "bwd_pre" in n)]
        if not fn or not wn:
            continue
        fb = statistics.median(fetch[fn[0]]) * 1024 * f_scale
        wb = statistics.median(write[wn[0]]) * 1024 * w_scale
        lines += [f"fetch_{key} = {fb:.0f}", f"write_{key} = {wb:.0f}", f"bytes_{key} = {fb + wb:.0f}"]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the steps, run one plain device copy of COPY_BYTES (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write profiles/long_context_hbm_traffic.txt from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the attention hot path here is "
              f"single-GPU and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    from workloads import WORKLOADS, digest, make_inputs
    w = WORKLOADS[4]
    inp = make_inputs(w)
    if args.copy_calibration:
        copy_calibration()
    step_ms, per, wall, (B, H, N, d) = run_gpu_bench(w, args.steps, args.warmup, inp)
    F = flops_fwd(B, H, N, d, w.causal)
    value = 3.5 * F / (step_ms * 1e-3) / 1e12

    dom = max(("fwd", "dkdv", "dq"), key=lambda n: per[n])
    ach = kernel_flops(dom, B, H, N, d, w.causal) / (per[dom] * 1e-3) / 1e12
    fwd_ach = kernel_flops("fwd", B, H, N, d, w.causal) / (per["fwd"] * 1e-3) / 1e12
    traffic = read_traffic()
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic.get(dom)}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0, 0.5) Q/K/V/dO, inputs resident in HBM)",
        "config": {"workload": "long-context: B=1 H=16 N=16384 d=128 bf16 causal, scale 1/sqrt(128)",
                   "B": B, "H": H, "N": N, "d": d, "causal": True, "input_sha256": digest(inp["q"], inp["k"], inp["v"])},
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "kernel_ms": {n: round(t, 4) for n, t in per.items()},
        "fwd_tflops": round(fwd_ach, 2), "fwd_pct_mfma_peak": round(100 * fwd_ach / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
