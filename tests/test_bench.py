"""Host-side logic of bench.py (no GPU): the flop and byte conventions of the
reported metric and the single-GPU guard."""
import math
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def test_long_context_flops_follow_the_metric_definition():
    w = WORKLOADS[4]
    f = bench.workload_fwd_flops(w, {})
    assert f == 4.0 * 1 * 16 * 16384 ** 2 * 128 / 2          # 4 B H N^2 d, halved for causal
    assert math.isclose(f / 1e12, 1.0995, rel_tol=1e-4)
    assert bench.kernel_flops("fwd", f) == f
    assert bench.kernel_flops("dkdv", f) == 2 * f and bench.kernel_flops("dq", f) == 1.5 * f
    # The metric counts the backward as 2.5 x forward (five products); the
    # two-kernel backward executes seven (S and dP in both dK/dV and dQ), so
    # the per-kernel figures are executed work, 3.5 x forward in total.
    assert bench.kernel_flops("dkdv", f) + bench.kernel_flops("dq", f) == 3.5 * f


def test_masked_workload_flops_scale_with_mask_and_padding():
    w3, w5 = WORKLOADS[3], WORKLOADS[5]
    kv = np.full(w3.B, 256, np.int32)
    assert bench.workload_fwd_flops(w3, {"kv_len": kv}) == 4.0 * w3.B * w3.H * w3.N * 256 * w3.d
    bm = np.zeros((w5.cells, w5.cells), np.uint8)
    bm[:, 0] = 1
    dense = 4.0 * w5.B * w5.H * w5.N ** 2 * w5.d
    assert math.isclose(bench.workload_fwd_flops(w5, {"block_mask": bm}), dense / w5.cells)


def test_compulsory_bytes():
    B, H, N, d = 1, 16, 16384, 128
    t, r = B * H * N * d * 2, B * H * N * 4
    assert bench.kernel_bytes("fwd", B, H, N, d, 2) == 4 * t + r          # Q, K, V in; O, lse out
    assert bench.kernel_bytes("dkdv", B, H, N, d, 2) == 6 * t + 2 * r     # Q, K, V, dO, lse, delta in; dK, dV out
    assert bench.kernel_bytes("dq", B, H, N, d, 2) == 6 * t + 2 * r       # Q, K, V, dO, O, lse in; dQ, delta out


def test_bound_from_arithmetic_intensity():
    w = WORKLOADS[4]
    f = bench.workload_fwd_flops(w, {})
    table = bench.kernel_table(w, {"fwd": 1.0, "dkdv": 2.0, "dq": 1.5}, f, 1, 16, 16384, 128)
    assert table["fwd"]["bound"] == "mfma" and table["dkdv"]["bound"] == "mfma"
    assert math.isclose(table["fwd"]["tflops"], f / 1e-3 / 1e12, rel_tol=1e-3)
    # the GPT-2 shape (N = 1024, d = 64, causal): the forward's intensity is below the ridge
    w2 = WORKLOADS[2]
    t2 = bench.kernel_table(w2, {"fwd": 0.03}, bench.workload_fwd_flops(w2, {}), w2.B, w2.H, w2.N, w2.d)
    assert t2["fwd"]["bound"] == "hbm"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_splitkv_pairs_and_bounds():
    """Allowed pairs under the bottom-right causal mask, against a brute-force
    count; decode is bandwidth-bound and chunked prefill matrix-bound."""
    from workloads import SPLITKV_WORKLOADS
    for Nq, Nk in ((1, 7), (3, 3), (5, 12), (9, 4)):
        i, j = np.arange(Nq)[:, None], np.arange(Nk)[None, :]
        assert bench.splitkv_pairs(Nq, Nk, True) == int((j <= i + Nk - Nq).sum())
        assert bench.splitkv_pairs(Nq, Nk, False) == Nq * Nk
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    f, b = bench.splitkv_alg(SPLITKV_WORKLOADS["decode"])
    assert f / b < ridge
    assert b == 2 * 256 * (2 + 2 * 16384) * 128 + 4 * 256
    f, b = bench.splitkv_alg(SPLITKV_WORKLOADS["prefill"])
    assert f / b > ridge


def test_profiled_kernel_names_exist_in_the_library():
    """The counter summary finds each kernel of the long-context step by the name
    rocprofv3 reports; every name bench.py looks for must be a kernel of the
    built library (a renamed template would otherwise drop out of the traffic
    figures)."""
    import shutil

    import pytest
    lib = os.path.join(ROOT, "exact_io_aware_flashattention_amd", "libfa.so")
    if not os.path.exists(lib) or shutil.which("nm") is None:
        pytest.skip("libfa.so not built or nm not available")
    syms = subprocess.run(["nm", "-C", lib], stdout=subprocess.PIPE, text=True, check=True).stdout
    for wl in bench.TRAFFIC_FILES:
        w = WORKLOADS[wl]
        for key, names in bench.stage_symbols(w.d, wl == 5).items():
            for sym in names:
                assert sym in syms, f"workload {wl} {key}: no kernel named {sym} in libfa.so"


def test_kernel_table_reports_median_min_and_measured_traffic():
    w = WORKLOADS[4]
    f = bench.workload_fwd_flops(w, {})
    per = {"fwd": 1.0, "dkdv": 2.0, "dq": 1.5}
    samples = {"fwd": [0.9, 1.0, 1.1], "dkdv": [2.0, 1.9, 2.1], "dq": [1.5, 1.6, 1.4]}
    table = bench.kernel_table(w, per, f, 1, 16, 16384, 128, samples, {"fwd": 8e8})
    assert table["fwd"]["ms_median"] == 1.0 and table["fwd"]["ms_min"] == 0.9
    assert math.isclose(table["fwd"]["hbm_gbs"], 8e8 / 1e-3 / 1e9, rel_tol=1e-3)
    assert "hbm_gbs" not in table["dq"]
    # dQ owes one product; it executes three (S and dP recomputed)
    assert math.isclose(table["dq"]["alg_tflops"] * 3, table["dq"]["tflops"], rel_tol=1e-3)
