"""Compile libfa.so for gfx950 with hipcc, in-tree.

Run as `python -m aware_attention_amd.build` (or through the repository's
build entry point). Always recompiles. Cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are kept out of every kernel.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc_command(out: str = LIB, extra=()) -> list[str]:
    return [HIPCC, *DEVICE_FLAGS, "-fPIC", "-shared", "-Wall",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, "fa_api.hip"), "-o", out, *extra]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
