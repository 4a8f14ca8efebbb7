"""Build libssmscan.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m mamba_selective_scan_ssm_amd.build
    python -m mamba_selective_scan_ssm_amd.build --poison-lds

Every HIP translation unit is compiled with packed-FP32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).  The second
form builds a debug library, _build/poison/libssmscan.so, whose kernels fill
their workgroup's LDS with NaN bit patterns at entry (SSM_POISON_LDS): run
the GPU parity tests against it (copied over the in-tree library) to catch a
read of LDS that nothing wrote first.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "ssmscan")
LIB = os.path.join(PKG, "libssmscan.so")
POISON_BUILD = os.path.join(ROOT, "_build", "poison")

SOURCES = ["api.cpp", "selective_scan.hip", "selective_scan_bwd.hip",
           "selective_scan_bwd_rows.hip", "ssd_chunk_scan.hip",
           "state_update.hip", "ssd_state_update.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libssmscan.so)")
    return path


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ([hipcc()] + common_flags() + [f"-D{d}" for d in defines] + lang +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed for {src}")
    return obj


def build_library(verbose: bool = False, poison_lds: bool = False) -> str:
    """Compile every source (always) and link libssmscan.so next to this file
    (poison_lds: the LDS-poisoning debug library under _build/poison)."""
    build_dir = POISON_BUILD if poison_lds else BUILD
    lib = os.path.join(POISON_BUILD, "libssmscan.so") if poison_lds else LIB
    defines = ("SSM_POISON_LDS",) if poison_lds else ()
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libssmscan.so failed")
    os.replace(tmp, lib)
    if verbose:
        print(lib)
    return lib


if __name__ == "__main__":
    build_library(verbose=True, poison_lds="--poison-lds" in sys.argv[1:])
