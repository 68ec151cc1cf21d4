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
# The timing-perturbed library for the race tests (-DFA_STRESS: pseudo-random
# pauses where waves hand LDS buffers to one another); loaded only when the
# environment variable AWARE_ATTENTION_LIB names it.
LIB_STRESS = os.path.join(PKG, "libfa_stress.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are kept out of every kernel.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Translation units of libfa.so: the forward entry points and host helpers,
# the backward entry points, the decode, the local pattern and the FP8 path.
# They compile in parallel, then link.
SOURCES = ["fa_api.hip", "fa_bwd_api.hip", "fa_decode_api.hip", "fa_local_api.hip",
           "fa_mx8_api.hip"]
_NOISE = "is not a recognized feature for this target"

# Per-source code generation flags. The backward's dK/dV kernel holds its dK
# and dV accumulators and its S and dP tiles at once (one wave per SIMD, up
# to 512 registers); with MFMA results placed in the accumulation registers
# by default, the register allocator shares them between the two and moves
# 128 accumulators out and back every tile. The vector-register form puts
# MFMA results in the arch VGPRs, so the accumulation registers hold the
# rest without copies.
SOURCE_FLAGS = {"fa_bwd_api.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc_compile(src: str, obj: str, extra=()) -> list[str]:
    return [HIPCC, *DEVICE_FLAGS, "-fPIC", "-c", "-Wall",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, src), "-o", obj, *extra]


def _messages(res) -> list[str]:
    return [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]


def build(verbose: bool = True, stress: bool = False) -> str:
    suffix = "_stress" if stress else ""
    objs = [os.path.join(CSRC, os.path.splitext(s)[0] + suffix + ".o") for s in SOURCES]
    extra = ["-DFA_STRESS"] if stress else []
    cmds = [hipcc_compile(s, o, [*extra, *SOURCE_FLAGS.get(s, [])]) for s, o in zip(SOURCES, objs)]
    procs = []
    for cmd in cmds:
        if verbose:
            print("[build]", " ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                      text=True))
    failed = []
    for cmd, proc in zip(cmds, procs):
        out, err = proc.communicate()
        res = subprocess.CompletedProcess(cmd, proc.returncode, out, err)
        msgs = _messages(res)
        if res.returncode != 0:
            failed.append("\n".join(msgs))
        elif verbose and msgs:
            print("\n".join(msgs), flush=True)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    lib = LIB_STRESS if stress else LIB
    tmp = lib + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", *objs, "-o", tmp]
    if verbose:
        print("[build]", " ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(_messages(res)))
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)
    return lib


if __name__ == "__main__":
    build(stress="--stress" in sys.argv[1:])
    sys.exit(0)
