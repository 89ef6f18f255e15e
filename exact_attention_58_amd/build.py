"""Builds the gfx950 HIP library libfa_mi355x.so in-tree with hipcc.

Usage: python -m exact_attention_58_amd.build [--resource-usage]
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa_mi355x.so")
SOURCES = [os.path.join(CSRC, "fa_fwd_kernels.hip"), os.path.join(CSRC, "fa_bwd_kernels.hip"),
           os.path.join(CSRC, "fa_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS]
    if resource_usage:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    cmd += ["-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is noise
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if msg.strip() and (verbose or resource_usage):
        print(msg)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose=True)
    print("built", LIB)
