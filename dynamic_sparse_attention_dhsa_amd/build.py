"""Build the gfx950 HIP libraries in place (hipcc, no JIT cache).

``libdhsa.so``: every DHSA translation unit, compiled for gfx950 only with
packed fp32 vector instructions disabled in device code, linked into one
shared library next to this file.  ``libdhsa_calib.so``: the calibration
kernels the benchmark measures the device's ceilings with (not part of the
DHSA C ABI).  ``python -m dynamic_sparse_attention_dhsa_amd.build`` rebuilds
both.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "libdhsa.so")
CALIB_LIB = os.path.join(PKG, "libdhsa_calib.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["api.cpp", "summarize.hip", "route.hip", "prefill_bf16.hip", "prefill_f32.hip", "chunking.hip", "decode.hip"]
CALIB_SOURCES = ["calib.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the DHSA library needs the ROCm toolchain to build")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


# Per-file flags.  The bf16 prefill kernel never meets a NaN (masked scores are -inf, weights are
# exponentials of finite or -inf values), so its max reductions need no signalling-NaN quieting:
# without IEEE mode each fmaxf is one v_max instead of two canonicalising moves and a v_max.
EXTRA_FLAGS = {"prefill_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + len(CALIB_SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES + CALIB_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
