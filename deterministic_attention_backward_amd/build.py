"""Build libattn_det.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m deterministic_attention_backward_amd.build [--resource-usage]

Builds libattn_det.so and its profiling twin libattn_det_profile.so (the same
sources with ATTN_PROFILE_WAIT=1: the main kernel also counts the cycles its
waves spend waiting for their dQ turn and at the hand-over barriers).
--resource-usage also asks the compiler for each kernel's register, LDS and
scratch (spill) usage and writes the remarks to _build/resource_usage.txt.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libattn_det.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.cpp", "bwd.hip", "fwd.hip", "probe.hip", "noalloc.hip"]
PROFILE_LIB_PATH = os.path.join(PKG_DIR, "libattn_det_profile.so")

# Packed-fp32 instructions are kept out of generated code on purpose.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def build(resource_usage: bool = False, verbose: bool = False, profile: bool = False) -> str:
    """Compile every source and link the shared library (or its profiling twin). Returns its path."""
    out_dir = os.path.join(PKG_DIR, "_build", "profile" if profile else "")
    os.makedirs(out_dir, exist_ok=True)
    lib_path = PROFILE_LIB_PATH if profile else LIB_PATH
    objs = []
    remarks = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(PKG_DIR, "..", "include"), "-c",
               os.path.join(CSRC, src), "-o", obj] + (["-DATTN_PROFILE_WAIT=1"] if profile else [])
        if resource_usage and src.endswith(".hip"):
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        if verbose:
            sys.stderr.write(res.stderr)
        if resource_usage:
            remarks.append(f"==== {src}\n" + "\n".join(
                ln for ln in res.stderr.splitlines() if "remark" in ln or "Function Name" in ln))
        objs.append(obj)
    tmp = lib_path + ".tmp"
    res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, lib_path)
    if resource_usage:
        with open(os.path.join(PKG_DIR, "_build", "resource_usage.txt"), "w") as f:
            f.write("\n".join(remarks) + "\n")
    return lib_path


def build_all(resource_usage: bool = False, verbose: bool = False) -> str:
    """The library and its profiling twin; returns the library's path."""
    path = build(resource_usage, verbose)
    build(False, verbose, profile=True)
    return path


if __name__ == "__main__":
    print(build_all(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv))
