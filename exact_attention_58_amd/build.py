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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compiles each source to an object (in parallel), then links the shared library."""
    tag = f".tmp{os.getpid()}"
    objs = [os.path.join(CSRC, os.path.basename(src) + tag + ".o") for src in SOURCES]
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is noise
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    out = []
    try:
        procs = [_run([HIPCC, *FLAGS, *extra, "-c", "-o", obj, src], verbose) for src, obj in zip(SOURCES, objs)]
        failed = []
        for src, p in zip(SOURCES, procs):
            text = p.communicate()[0]
            out.append(text)
            if p.returncode != 0:
                failed.append(src)
        msg = "\n".join(l for l in "\n".join(out).splitlines() if not any(n in l for n in noise))
        if failed:
            raise RuntimeError(f"hipcc failed on {failed}:\n{msg}")
        if msg.strip() and (verbose or resource_usage):
            print(msg)
        tmp = LIB + tag
        link = _run([HIPCC, *FLAGS, "-o", tmp, *objs], verbose)
        text = link.communicate()[0]
        if link.returncode != 0:
            raise RuntimeError(f"link failed ({link.returncode}):\n{text}")
        os.replace(tmp, LIB)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose=True)
    print("built", LIB)
