"""Build the HIP library ``libringattn.so`` in-tree for gfx950.

Every source under ``csrc/`` is compiled by hipcc into ``_build/`` at the
repository root and linked into ``blockwise_ring_attention_amd/libringattn.so``.
Runs on a host without a GPU (hipcc cross-compiles).  Usage::

    python -m blockwise_ring_attention_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libringattn.so")

SOURCES = ["api.cpp", "emulator.cpp", "elementwise.hip", "fwd_fp32.hip",
           "fwd_bf16.hip", "bwd_bf16.hip", "decode_bf16.hip",
           "ffn_bf16.hip"]

ARCH = "gfx950"
# Packed fp32 VALU instructions are disabled on purpose for every HIP source.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wno-inline-asm",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


# roctx ranges (ring steps in the emulator) come from the profiler SDK's
# marker library, part of ROCm.
LINK = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx"]


# Per-source flags.  The backward kernels keep the MFMA results that vector
# code reads (scores) in VGPRs; their long-lived accumulators are placed in
# AGPRs explicitly (inline asm), so the MFMA builtins are told to use VGPRs.
SOURCE_FLAGS = {"bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the device-only feature
    out = "\n".join(l for l in p.stdout.splitlines() if "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc, *FLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, *LINK, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
