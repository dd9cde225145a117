"""Compile the HIP sources into libfa.so (gfx950) next to this file.

Every call recompiles.  Object files go to ``_build/``; the translation units
are compiled in parallel.  All HIP code is built with packed-FP32 VALU ops
disabled, so the compiler never emits v_pk_{add,mul,fma}_f32.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_bf16.hip", "fa_split.hip", "fa_decode.hip", "fa_fp8.hip"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", f"-I{INCLUDE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(jobs: int = 4, extra_flags=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    cc = hipcc()
    cmds = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
