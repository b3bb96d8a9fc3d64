"""Compile libmrope_attn.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m diffusion_transformer_image_head_amd.build [--verbose]``.
The library is written next to this file; the binding loads it from there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmrope_attn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def flags(resource_usage: bool = False) -> list:
    f = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU forms stay disabled (see the HIP toolchain notes)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]
    if resource_usage:
        f += ["-Rpass-analysis=kernel-resource-usage"]
    return f


def build(verbose: bool = False) -> str:
    """Compile the shared library; returns its path. Always recompiles."""
    src = os.path.join(CSRC, "mrope_attn.hip")
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags(resource_usage=verbose) + [src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
