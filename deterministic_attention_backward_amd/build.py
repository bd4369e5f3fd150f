"""Build libattn_det.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m deterministic_attention_backward_amd.build [--resource-usage]

--resource-usage also asks the compiler for each kernel's register, LDS and
scratch (spill) usage and writes the remarks next to the library as
resource_usage.txt.
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
SOURCES = ["api.cpp", "bwd.hip", "fwd.hip"]

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


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every source and link the shared library. Returns its path."""
    out_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    remarks = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(PKG_DIR, "..", "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
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
    tmp = LIB_PATH + ".tmp"
    res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB_PATH)
    if resource_usage:
        with open(os.path.join(PKG_DIR, "_build", "resource_usage.txt"), "w") as f:
            f.write("\n".join(remarks) + "\n")
    return LIB_PATH


if __name__ == "__main__":
    path = build(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv)
    print(path)
