"""Compiled-code check of the tile loops (CPU: compiles the HIP sources to
gfx950 assembly, runs nothing).

Each tile loop starts by waiting for the tile loads it requested one tile
earlier, synchronises the work-group, then requests the next tile.  Vector
memory waits count outstanding loads in order, so any further wait on vector
memory between that request and the tile's matrix products also waits for the
next tile's data: the request is then no longer ahead of the work, and every
tile pays the whole load latency.  The compiler inserts such waits by itself
when a register load it tracks (row statistics, or fragments loaded before the
loop) is still outstanding where a product needs it.  This test compiles the
kernels and fails if a wait of that kind sits between a tile request and the
next product of the hot instances (bf16 forward, dQ and dK/dV without block
mask or dropout; the FP8 forward).  The intended tile-start wait is the one
followed by the empty compiler barrier that the kernels place after it, or the
inline-assembly form.
"""
import os
import re
import shutil
import subprocess

import pytest

from exact_io_aware_flashattention_amd import _build

pytestmark = pytest.mark.timeout(600)


def _have_hipcc():
    try:
        return bool(_build.hipcc())
    except RuntimeError:
        return False


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not _have_hipcc():
        pytest.skip("hipcc not available")
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in ("fa_bf16.hip", "fa_fp8.hip"):
        path = os.path.join(str(d), src + ".s")
        cmd = [_build.hipcc(), *_build.COMMON, "--cuda-device-only", "-S", "-o", path,
               os.path.join(_build.CSRC, src)]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-2000:]
        out[src] = open(path).read()
    return out


def kernel_body(text, symbol):
    start = text.index(symbol + ":")
    end = text.index(".Lfunc_end", start)
    return [l.strip() for l in text[start:end].split("\n")]


def waits_behind_tile_request(lines):
    """Indices of vector-memory waits that sit between a tile-load request
    and the next matrix product, before any barrier, and are not the
    intended tile-start wait."""
    issued = False
    pending = None
    bad = []
    for i, l in enumerate(lines):
        if "offen lds" in l:          # a tile-load request (buffer load into LDS)
            issued, pending = True, None
        elif l.startswith("s_barrier"):
            issued, pending = False, None
        elif issued and l.startswith("s_waitcnt") and "vmcnt" in l:
            intended = (i > 0 and lines[i - 1] == ";;#ASMSTART") or \
                any(x == ";;#ASMSTART" for x in lines[i + 1:i + 3])
            pending = None if intended else i
        elif pending is not None and l.startswith("v_mfma"):
            bad.append(pending)
            pending = None
    return bad


HOT = [
    ("fa_bf16.hip", f"_ZN2fa15fwd_bf16_kernelILi{d}ELi0EEEvNS_8AttnArgsE") for d in (64, 96, 128)
] + [
    ("fa_bf16.hip", f"_ZN2fa14dq_bf16_kernelILi{d}ELi0EEEvNS_8AttnArgsE") for d in (64, 96, 128)
] + [
    ("fa_bf16.hip", f"_ZN2fa16dkdv_bf16_kernelILi{d}ELi0ELb0EEEvNS_8AttnArgsE") for d in (64, 96, 128)
] + [
    ("fa_fp8.hip", f"_ZN2fa12_GLOBAL__N_114fwd_fp8_kernelILi{d}EEEvNS_8AttnArgsE") for d in (64, 128)
]


@pytest.mark.parametrize("src,symbol", HOT, ids=[s.split("kernel")[0][6:] + s.split("ILi")[1][:3] for _, s in HOT])
def test_no_wait_behind_tile_request(asm, src, symbol):
    lines = kernel_body(asm[src], symbol)
    assert any("offen lds" in l for l in lines), "no tile-load request found"
    assert any(l.startswith("v_mfma") for l in lines), "no matrix product found"
    bad = waits_behind_tile_request(lines)
    assert not bad, f"{symbol}: vector-memory waits between a tile request and a product at lines " \
                    f"{bad[:5]}: " + " | ".join(lines[i] for i in bad[:3])


def test_scan_flags_a_planted_wait():
    # the scan itself: a compiler-style wait after a request and before a
    # product is reported; the tile-start form and waits after a barrier are not
    body = ["buffer_load_dwordx4 v1, s[0:3], 0 offen lds", "s_waitcnt vmcnt(0)", "v_mfma_f32_32x32x16_bf16 a",
            "s_waitcnt vmcnt(0)", ";;#ASMSTART", ";;#ASMEND", "s_barrier",
            "s_waitcnt vmcnt(0)", "v_mfma_f32_32x32x16_bf16 b",
            "buffer_load_dwordx4 v1, s[0:3], 0 offen lds", "s_waitcnt vmcnt(0)", ";;#ASMSTART", ";;#ASMEND",
            "v_mfma_f32_32x32x16_bf16 c"]
    assert waits_behind_tile_request(body) == [1]
