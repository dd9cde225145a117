"""Benchmark of the attention hot path on one MI355X.

One step = one forward (fa_fwd) and one backward (fa_bwd's two stages: dQ
with the row terms delta = rowsum(dO * O) formed in the same kernel, then
dK/dV) over the long-context workload: B=1, H=16,
N=16384, d=128, bf16, causal, scale 1/sqrt(128), Q/K/V/dO ~ N(0, 0.5) from the
seeded generator.  Inputs are resident in HBM before timing starts.

value = attention TFLOP/s of fwd+bwd = 3.5 * F_fwd / t_step with
F_fwd = 4 B H N^2 d / 2 (causal), i.e. backward counted as 2.5x forward.

Each stage is bracketed by HIP events recorded on the stream the library
launches on, so the per-kernel averages come from the timed steps themselves.
The roofline object describes the kernel with the largest average time.

cpu_baseline times the fp64 CPU oracle (forward + backward) on six heads of
the same workload (about 10-30 s on one host).

--workload K times one of the other workloads (1 tiny fp32, 2 GPT-2 shaped,
3 BERT-shaped with key padding, 5 block-sparse 64K, 6 long context at head
dimension 256) with the same step and
prints the same kind of line (no CPU leg unless --cpu-baseline is given); the
default line is the long-context workload.  Per kernel it reports achieved
TFLOP/s against the bf16 matrix peak and achieved GB/s of compulsory HBM
traffic against 8 TB/s ("alg_gbs": compulsory bytes / time, a derived
figure), and names the bound of each kernel from its arithmetic intensity
(compulsory bytes) against the ridge point.  Where a counter summary for the
workload is committed under profiles/ and still matches the kernel sources,
each kernel also gets "hbm_bytes" (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled
by a plain copy's readings) and "hbm_gbs" = hbm_bytes / time.

Every per-kernel time is reported as the mean over the timed steps, with the
median and the minimum beside it.  --cold writes a 512 MiB scrub buffer before
every timed launch (outside its event bracket), so each kernel starts with its
operands evicted from L2 and the MALL; the step time is then the sum of the
kernels' times.
"""
from __future__ import annotations

import argparse
import gc
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
PEAK_F32_TFLOPS = 157.3        # fp32 matrix peak
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 matrix peak


def _gc_pause():
    """Collect now and keep Python's cyclic collector off while the timed launches
    are enqueued: a full collection (tens of ms with torch loaded) can stall the
    launching thread long enough for the GPU queue to drain, and the idle time
    would be counted in whichever kernel's event interval was open."""
    gc.collect()
    gc.disable()


def _gc_resume():
    gc.enable()


def flops_fwd(B, H, N, d, causal, cell_frac=1.0):
    f = 4.0 * B * H * N * N * d * cell_frac
    return f / 2 if causal else f


def workload_fwd_flops(w, inp):
    """Forward attention flops of a workload: 4 B H N^2 d, halved for causal,
    scaled by the fraction of nonzero mask cells and by mean(kv_len) / N."""
    import numpy as np
    f = flops_fwd(w.B, w.H, w.N, w.d, w.causal)
    if inp.get("block_mask") is not None:
        f *= float(np.asarray(inp["block_mask"]).sum()) / w.cells ** 2
    if inp.get("kv_len") is not None:
        f *= float(np.minimum(np.asarray(inp["kv_len"]), w.N).mean()) / w.N
    return f


PRODUCTS = {"fwd": 2, "dkdv": 4, "dq": 3}
# Products each kernel owes the method (dQ = scale dS K is one product; S and
# dP are recomputed in the dQ kernel, which the executed count includes).
ALG_PRODUCTS = {"fwd": 2, "dkdv": 4, "dq": 1}


def kernel_flops(name, f_fwd):
    """GEMM flops a kernel executes per launch: score entries x 2d per product,
    fwd 2 products (S, PV), dkdv 4 (S, dP, dV, dK), dq 3 (S, dP, dQ)."""
    return PRODUCTS[name] * f_fwd / 2


def kernel_bytes(name, B, H, N, d, esize):
    """Compulsory HBM bytes per launch (each operand read once, each output
    written once): the IO lower bound of the pages' complexity analysis.  The
    dQ stage reads Q, K, V, dO, O and lse and writes dQ and delta."""
    t, r = B * H * N * d * esize, B * H * N * 4
    return {"fwd": 3 * t + t + r, "dkdv": 4 * t + 2 * r + 2 * t, "dq": 5 * t + r + t + r}[name]


def run_gpu_bench_dropout(w, steps, warmup, inp, p, seed=2024):
    """Step with dropout on P: fa_fwd_dropout + fa_bwd_dropout (the backward's
    stages are one call), each bracketed by HIP events on the launch stream."""
    import numpy as np
    import torch

    import exact_io_aware_flashattention_amd as fa

    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(inp[n]).to(dev, torch.bfloat16) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bm = None if inp.get("block_mask") is None else torch.from_numpy(np.ascontiguousarray(inp["block_mask"])).to(dev)
    kl = None if inp.get("kv_len") is None else torch.from_numpy(inp["kv_len"].astype(np.int32)).to(dev)
    ws = torch.empty(max(fa.fa_bwd_workspace_bytes(B, H, N, d, fa.FA_BF16, bm is not None), 256),
                     dtype=torch.uint8, device=dev)
    kw = dict(scale=w.scale, causal=w.causal, block_mask=bm, kv_len=kl, dropout_p=p, seed=seed)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, stream=stream, **kw)
        if ev:
            ev[1].record(stream)
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, workspace=ws, stream=stream, **kw)
        if ev:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _gc_pause()
    start.record(stream)
    for i in range(steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    _gc_resume()
    per = {"fwd": sum(e[0].elapsed_time(e[1]) for e in evs) / steps,
           "bwd": sum(e[1].elapsed_time(e[2]) for e in evs) / steps}
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(dq).all())
    return start.elapsed_time(end) / steps, per, (B, H, N, d)


SCRUB_BYTES = 512 << 20


def run_gpu_bench(w, steps, warmup, inp, cold=False):
    import numpy as np
    import torch

    import exact_io_aware_flashattention_amd as fa

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, do = (torch.from_numpy(inp[n]).to(dev, tdt) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    bm = None if inp.get("block_mask") is None else torch.from_numpy(np.ascontiguousarray(inp["block_mask"])).to(dev)
    kl = None if inp.get("kv_len") is None else torch.from_numpy(inp["kv_len"].astype(np.int32)).to(dev)
    ws_bytes = fa.fa_bwd_dkdv_workspace_bytes(N, d, fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32, bm is not None)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev) if ws_bytes else None
    kw = dict(scale=w.scale, causal=w.causal, block_mask=bm, kv_len=kl)
    stream = torch.cuda.current_stream()
    scrub = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev) if cold else None
    launches = [lambda: fa.fa_fwd(q, k, v, o, lse, stream=stream, **kw),
                lambda: fa.fa_bwd_dq_delta(q, k, v, o, do, lse, delta, dq, stream=stream, **kw),
                lambda: fa.fa_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, workspace=ws, stream=stream, **kw)]

    def step(ev=None):
        for j, launch in enumerate(launches):
            if scrub is not None:
                scrub.fill_(float(j))     # evict the operands: 512 MiB written through L2 and the MALL
            if ev:
                ev[2 * j].record(stream)
            launch()
            if ev:
                ev[2 * j + 1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(launches))] for _ in range(steps)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    _gc_pause()
    start.record(stream)
    for i in range(steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    _gc_resume()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    names = ["fwd", "dq", "dkdv"]
    samples = {n: [ev[2 * j].elapsed_time(ev[2 * j + 1]) for ev in evs] for j, n in enumerate(names)}
    per = {n: sum(s) / steps for n, s in samples.items()}      # mean ms per launch
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(dq).all())
    step_ms = sum(per.values()) if cold else total_ms / steps
    return step_ms, per, wall, (B, H, N, d), samples


def splitkv_pairs(Nq, Nk, causal):
    """Allowed (query, key) pairs of one head: all Nq Nk, or under the causal
    mask aligned to the last Nq keys (j <= i + Nk - Nq) sum_i min(Nk, i + Nk - Nq + 1)."""
    if not causal:
        return Nq * Nk
    return sum(max(0, min(Nk, i + Nk - Nq + 1)) for i in range(Nq))


def splitkv_alg(w, fp8kv=False):
    """Algorithmic flops (S and PV products over allowed pairs) and compulsory
    HBM bytes (Q, K, V read once; O and lse written once) of one split-key
    forward call; fp8kv: K and V are one byte per feature."""
    B, H, Nq, Nk, d = w["B"], w["H"], w["Nq"], w["Nk"], w["d"]
    flops = 4.0 * B * H * splitkv_pairs(Nq, Nk, w["causal"]) * d
    nbytes = B * H * (2 * 2 * Nq + (1 if fp8kv else 2) * 2 * Nk) * d + 4 * B * H * Nq
    return flops, nbytes


def run_gpu_bench_splitkv(which, steps, warmup, fp8kv=False):
    """One step = one fa_fwd_splitkv call (range kernel + merge), bracketed by
    HIP events on the launch stream; fp8kv: fa_fwd_splitkv_fp8kv with K and V
    quantized per tensor to E4M3 (decode only)."""
    import torch

    import exact_io_aware_flashattention_amd as fa
    from workloads import SPLITKV_WORKLOADS, draw_split_qkv, digest

    w = SPLITKV_WORKLOADS[which]
    B, H, Nq, Nk, d = w["B"], w["H"], w["Nq"], w["Nk"], w["d"]
    qa, ka, va = draw_split_qkv(B, H, Nq, Nk, d, w["sigma"], w["seed"])
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(a).to(dev, torch.bfloat16) for a in (qa, ka, va))
    if fp8kv:
        from workloads import quantize_e4m3
        (k8, dk), (v8, dv) = quantize_e4m3(ka), quantize_e4m3(va)
        k, v = torch.from_numpy(k8).to(dev), torch.from_numpy(v8).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    scale = 1.0 / math.sqrt(d)

    def step():
        if fp8kv:
            fa.fa_fwd_splitkv_fp8kv(q, k, v, float(dk), float(dv), o, lse, scale=scale, causal=w["causal"],
                                    workspace=ws, stream=stream)
        else:
            fa.fa_fwd_splitkv(q, k, v, o, lse, scale=scale, causal=w["causal"], workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _gc_pause()
    start.record(stream)
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    _gc_resume()
    assert bool(torch.isfinite(o).all())
    call_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    flops, nbytes = splitkv_alg(w, fp8kv)
    nsplit = fa.fa_fwd_splitkv_num_splits(B, H, Nq, Nk, 0)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    tf, gbs = flops / (call_ms * 1e-3) / 1e12, nbytes / (call_ms * 1e-3) / 1e9
    if flops / nbytes > ridge:
        metric, value, unit = "split-key forward TFLOP/s (bf16, 1 GPU)", tf, "TFLOP/s"
        roofline = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    else:
        metric, value, unit = (f"split-key forward GB/s of compulsory HBM traffic "
                               f"({'bf16 queries, E4M3 K/V' if fp8kv else 'bf16'}, 1 GPU)", gbs, "GB/s")
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roofline.update({"kernel": "fa_fwd_splitkv call (range kernel + merge)", "traffic": None,
                     "alg_flops": flops, "alg_bytes": nbytes})
    return {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(start.elapsed_time(end) / steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 queries, E4M3 K/V" if fp8kv else "bf16",
        "data": f"synthetic (seeded N(0, {w['sigma'] ** 2:g}) Q/K/V, inputs resident in HBM)",
        "config": {"workload": w["desc"] + (", K/V cache in E4M3" if fp8kv else ""), "B": B, "H": H, "Nq": Nq,
                   "Nk": Nk, "d": d, "causal": w["causal"],
                   "num_splits": nsplit, "input_sha256": digest(qa, ka, va)},
        "call_ms": round(call_ms, 4), "tflops": round(tf, 2), "alg_gbs": round(gbs, 1),
        "roofline": roofline}


def run_gpu_bench_fp8(w, steps, warmup, inp):
    """One step = one fa_fwd_fp8 call on the workload's Q, K, V quantized per
    tensor to E4M3 (descale = amax / 448), bracketed by HIP events on the
    launch stream."""
    import torch

    import exact_io_aware_flashattention_amd as fa
    from workloads import quantize_e4m3

    dev = torch.device("cuda:0")
    (q8, dq), (k8, dk), (v8, dv) = (quantize_e4m3(inp[n]) for n in ("q", "k", "v"))
    q, k, v = (torch.from_numpy(x).to(dev) for x in (q8, k8, v8))
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        fa.fa_fwd_fp8(q, k, v, float(dq), float(dk), float(dv), o, lse, scale=w.scale, causal=w.causal,
                      stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _gc_pause()
    start.record(stream)
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    _gc_resume()
    assert bool(torch.isfinite(o.float()).all())
    call_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    return start.elapsed_time(end) / steps, call_ms, (B, H, N, d)


COPY_BYTES = 256 << 20

DESC = {1: "tiny exact: B=1 H=2 N=128 d=64 fp32, scale 1/8",
        2: "GPT-2 shaped: B=8 H=12 N=1024 d=64 bf16 causal, scale 1/8",
        3: "BERT-large shaped: B=32 H=16 N=512 d=64 bf16, key padding kv_len ~ U[128, 512], scale 1/8",
        4: "long-context: B=1 H=16 N=16384 d=128 bf16 causal, scale 1/sqrt(128)",
        5: "block-sparse: B=1 H=8 N=65536 d=64 bf16, 128x128 cell mask (band, 2 random cells per row, "
           "first column), scale 1/8",
        6: "long-context, head dim 256: B=1 H=8 N=16384 d=256 bf16 causal, scale 1/16",
        7: "long-context, head dim 96: B=1 H=16 N=16384 d=96 bf16 causal, scale 1/sqrt(96)",
        8: "long-context, head dim 160: B=1 H=16 N=16384 d=160 bf16 causal, scale 1/sqrt(160)"}


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


def cpu_baseline(w, inp, heads=6):
    """fp64 oracle fwd + bwd on heads 0..heads-1 of batch entry 0 (all rows, all keys)."""
    import numpy as np

    from oracle import sparse
    cores = len(os.sched_getaffinity(0))
    kv = None if inp.get("kv_len") is None else int(inp["kv_len"][0])
    kw = dict(causal=w.causal, block_mask=inp.get("block_mask"), kv_len=kv)
    t0 = time.perf_counter()
    for h in range(heads):
        Q, K, V, dO = (inp[n][0, h].astype(np.float64) for n in ("q", "k", "v", "do"))
        sparse.head_forward(Q, K, V, w.scale, **kw)
        sparse.head_backward(Q, K, V, dO, w.scale, **kw)
    dt = time.perf_counter() - t0
    f = 3.5 * workload_fwd_flops(w, inp) * heads / (w.B * w.H)
    return {"value": round(f / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"heads 0-{heads - 1} of batch entry 0 ({heads} of {w.B * w.H} heads) of the same workload "
                      f"(N={w.N}, d={w.d}), fp64 forward+backward, {dt:.1f} s",
            "seconds": round(dt, 2)}


PROFILES = os.path.join(ROOT, "profiles")
# Counter summaries per workload, and the kernels each stage of a step launches
# (a stage's bytes are the sum over its kernels; the block-mask dK/dV stage
# also runs the split count and plan kernels).
TRAFFIC_FILES = {2: "gpt2_shaped_hbm_traffic.txt", 3: "bert_shaped_hbm_traffic.txt",
                 4: "long_context_hbm_traffic.txt", 5: "block_sparse_hbm_traffic.txt"}
TRAFFIC_FILE = os.path.join(PROFILES, TRAFFIC_FILES[4])


def stage_symbols(d, block_mask):
    split = "true" if block_mask else "false"
    return {"fwd": [f"fwd_bf16_kernel<{d}, 0>"],
            "dkdv": [f"dkdv_bf16_kernel<{d}, 0, {split}>"] + (["split_count_kernel", "split_plan_kernel"]
                                                               if block_mask else []),
            "dq": [f"dq_bf16_kernel<{d}, 0>"]}


def kernel_source_hash():
    """SHA-256 over the HIP sources; counter readings are only reported while it matches."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_io_aware_flashattention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def read_traffic(workload=4):
    """HBM bytes per launch from the committed counter summary of a workload,
    or {} when there is none or the kernels changed after it was taken."""
    path = os.path.join(PROFILES, TRAFFIC_FILES.get(workload, "-"))
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return {}
    return {k[len("bytes_"):]: float(v) for k, v in kv.items() if k.startswith("bytes_")}


def summarize_counters(fetch_csv, write_csv, command, workload=4):
    """Write a workload's per-kernel HBM traffic summary from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch).  Each counter is scaled by
    its reading for the plain copy of COPY_BYTES made by --copy-calibration."""
    import csv
    import statistics

    from workloads import WORKLOADS
    w = WORKLOADS[workload]
    symbols = stage_symbols(w.d, workload == 5)

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
    lines = [f"# HBM traffic per launch, {DESC[workload]}",
             f"# command: {command}",
             f"# calibration: a {COPY_BYTES >> 20} MiB device copy reads FETCH_SIZE {max(fetch[copy_name]):.1f} KiB "
             f"(scale {f_scale:.4f}) and WRITE_SIZE {max(write[copy_name]):.1f} KiB (scale {w_scale:.4f})",
             f"source_hash = {kernel_source_hash()}",
             f"fetch_scale = {f_scale:.6f}", f"write_scale = {w_scale:.6f}"]
    for key, syms in symbols.items():
        fb = wb = 0.0
        for sym in syms:
            fn = [n for n in fetch if sym in n]
            wn = [n for n in write if sym in n]
            if len(fn) != 1 or len(wn) != 1:
                raise SystemExit(f"{key}: kernel {sym} matches {fn} in the counter files; names: {sorted(fetch)}")
            fb += statistics.median(fetch[fn[0]]) * 1024 * f_scale
            wb += statistics.median(write[wn[0]]) * 1024 * w_scale
        lines += [f"fetch_{key} = {fb:.0f}", f"write_{key} = {wb:.0f}", f"bytes_{key} = {fb + wb:.0f}"]
    with open(os.path.join(PROFILES, TRAFFIC_FILES[workload]), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def kernel_table(w, per, f_fwd, B, H, N, d, samples=None, traffic=None):
    """Per-kernel achieved TFLOP/s (executed products; for dQ also its one
    algorithmic product), compulsory-traffic GB/s ("alg_gbs"), the bound implied
    by arithmetic intensity (flops per compulsory byte) against the ridge point
    peak_flops / peak_bandwidth, and, with a matching counter summary, the
    measured HBM bytes and GB/s."""
    import statistics
    esize = 2 if w.dtype == "bf16" else 4
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    out = {}
    for n, ms in per.items():
        fl, by = kernel_flops(n, f_fwd), kernel_bytes(n, B, H, N, d, esize)
        row = {"ms": round(ms, 4)}
        if samples:
            row["ms_median"] = round(statistics.median(samples[n]), 4)
            row["ms_min"] = round(min(samples[n]), 4)
        row.update({"tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                    "alg_gbs": round(by / (ms * 1e-3) / 1e9, 1), "alg_bytes": by,
                    "bound": "mfma" if fl / by > ridge else "hbm"})
        if ALG_PRODUCTS[n] != PRODUCTS[n]:
            row["alg_tflops"] = round(ALG_PRODUCTS[n] * f_fwd / 2 / (ms * 1e-3) / 1e12, 2)
        if traffic and n in traffic:
            row["hbm_bytes"] = traffic[n]
            row["hbm_gbs"] = round(traffic[n] / (ms * 1e-3) / 1e9, 1)
        out[n] = row
    return out


def sweep(steps, warmup):
    """The metric's N = 1K..16K range: N in {1K, 2K, 4K, 8K, 16K} with B = 16K / N,
    H = 16, d in {64, 128}, causal off and on, bf16, scale 1/sqrt(d); Q/K/V/dO
    i.i.d. N(0, 1) from one seeded draw (seed 6) per d, reshaped (B N is the
    same for every N).  One JSON line per configuration."""
    import numpy as np

    from workloads import Workload, draw_qkvdo
    for d in (64, 128):
        flat = draw_qkvdo(1, 16, 16384, d, "bf16", 1.0, 6)
        for N in (1024, 2048, 4096, 8192, 16384):
            B = 16384 // N
            inp = {n: a.reshape(B, 16, N, d) for n, a in zip(("q", "k", "v", "do"), flat)}
            for causal in (False, True):
                w = Workload(0, "sweep", B, 16, N, d, "bf16", causal, 1.0 / math.sqrt(d), 1.0)
                step_ms, per, _, _, _ = run_gpu_bench(w, steps, warmup, inp)
                F = workload_fwd_flops(w, inp)
                t_bwd = per["dkdv"] + per["dq"]
                line = {"B": B, "H": 16, "N": N, "d": d, "causal": causal, "ms_per_step": round(step_ms, 4),
                        "fwd_bwd_tflops": round(3.5 * F / (step_ms * 1e-3) / 1e12, 1),
                        "fwd_tflops": round(F / (per["fwd"] * 1e-3) / 1e12, 1),
                        "bwd_tflops": round(2.5 * F / (t_bwd * 1e-3) / 1e12, 1),
                        "kernel_ms": {n: round(t, 4) for n, t in per.items()}}
                print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, choices=(1, 2, 3, 4, 5, 6, 7, 8),
                    help="workload to time (default 4, the long-context line)")
    ap.add_argument("--sweep", action="store_true", help="time the N = 1K..16K sweep (one JSON line per shape)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="time the step with dropout on P at this rate (fa_fwd_dropout + fa_bwd_dropout)")
    ap.add_argument("--splitkv", choices=("decode", "prefill"),
                    help="time the split-key forward (fa_fwd_splitkv) on a decode or chunked-prefill shape")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward (fa_fwd_fp8) on the workload's inputs quantized to E4M3")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg (profiling runs)")
    ap.add_argument("--cpu-baseline", action="store_true", help="run the CPU oracle leg for --workload other than 4")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the steps, run one plain device copy of COPY_BYTES (counter calibration)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB scrub buffer before every timed launch (cold L2 and MALL)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write the --workload's HBM traffic summary under profiles/ from two rocprofv3 --pmc runs "
                         "and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, workload=args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the attention hot path here is "
              f"single-GPU and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep(args.steps, args.warmup)
        return
    if args.splitkv:
        if args.fp8 and args.splitkv != "decode":
            print("--fp8 with --splitkv applies to decode only (an E4M3 key/value cache)", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(run_gpu_bench_splitkv(args.splitkv, args.steps, args.warmup, fp8kv=args.fp8)), flush=True)
        return

    from workloads import WORKLOADS, digest, make_inputs
    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    if args.fp8:
        step_ms, call_ms, (B, H, N, d) = run_gpu_bench_fp8(w, args.steps, args.warmup, inp)
        F = workload_fwd_flops(w, inp)
        tf = F / (call_ms * 1e-3) / 1e12
        print(json.dumps({
            "metric": "FP8 attention forward TFLOP/s (E4M3 inputs, 1 GPU)", "value": round(tf, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8-e4m3", "data": f"synthetic (seeded N(0, {w.sigma ** 2:g}) Q/K/V quantized per tensor "
                                          f"to E4M3, inputs resident in HBM)",
            "config": {"workload": f"workload {args.workload}, forward on E4M3 inputs", "B": B, "H": H, "N": N,
                       "d": d, "causal": w.causal},
            "roofline": {"bound": "mfma", "kernel": "fwd_fp8_kernel", "achieved": round(tf, 2),
                         "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                         "traffic": None}}), flush=True)
        return
    if args.dropout:
        step_ms, per, (B, H, N, d) = run_gpu_bench_dropout(w, args.steps, args.warmup, inp, args.dropout)
        F = workload_fwd_flops(w, inp)
        t = round(args.dropout * 256)
        print(json.dumps({
            "metric": METRIC, "value": round(3.5 * F / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": f"synthetic (seeded N(0, {w.sigma ** 2:g}) Q/K/V/dO, inputs resident in HBM)",
            "config": {"workload": f"workload {args.workload} with dropout p = {t}/256 on P", "B": B, "H": H,
                       "N": N, "d": d, "causal": w.causal},
            "kernel_ms": {n: round(x, 4) for n, x in per.items()},
            "fwd_tflops": round(F / (per["fwd"] * 1e-3) / 1e12, 2),
            "bwd_tflops": round(2.5 * F / (per["bwd"] * 1e-3) / 1e12, 2)}), flush=True)
        return
    if args.copy_calibration:
        copy_calibration()
    step_ms, per, wall, (B, H, N, d), samples = run_gpu_bench(w, args.steps, args.warmup, inp, cold=args.cold)
    F = workload_fwd_flops(w, inp)
    value = 3.5 * F / (step_ms * 1e-3) / 1e12
    traffic = {} if args.cold else read_traffic(args.workload)
    table = kernel_table(w, per, F, B, H, N, d, samples, traffic)

    dom = max(("fwd", "dkdv", "dq"), key=lambda n: per[n])
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    if table[dom]["bound"] == "mfma":
        ach = table[dom]["tflops"]
        roofline = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4)}
    else:
        ach = table[dom]["alg_gbs"]
        roofline = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4)}
    roofline["traffic"] = traffic.get(dom)
    config = {"workload": DESC[args.workload], "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
              "input_sha256": digest(inp["q"], inp["k"], inp["v"])}
    if args.cold:
        config["cold"] = "512 MiB scrub before every launch; step = sum of kernel times"
    if inp.get("block_mask") is not None:
        config["mask_cells"] = int(inp["block_mask"].sum())
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": f"synthetic (seeded N(0, {w.sigma ** 2:g}) Q/K/V/dO, inputs resident in HBM)",
        "config": config,
        "pct_mfma_peak": round(100 * value / peak, 2),
        "kernel_ms": {n: round(t, 4) for n, t in per.items()},
        "fwd_tflops": table["fwd"]["tflops"], "fwd_pct_mfma_peak": round(100 * table["fwd"]["tflops"] / peak, 2),
        "kernels": table,
        "roofline": roofline,
    }
    if (args.workload == 4 and not args.no_cpu_baseline) or args.cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
