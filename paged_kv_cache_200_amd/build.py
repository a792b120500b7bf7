"""Build libpkv.so (HIP kernels for gfx950 + host block manager) in-tree.

    python -m paged_kv_cache_200_amd.build [--verbose]

Each ``csrc/*.hip`` file is compiled by hipcc for gfx950 only; the host-only
block manager by g++; everything is linked into
``paged_kv_cache_200_amd/libpkv.so``.  Packed fp32 instructions are disabled
in device code.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"

HIP_SOURCES = ["paged_decode.hip", "prefill.hip", "kv_append.hip", "copy_blocks.hip",
               "status.hip", "static_scratch.hip"]
HOST_SOURCES = ["block_manager.cpp", "replay.cpp", "decode_layers.cpp"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm installation is required to build libpkv")


def _extra_flags():
    """Extra hipcc flags from PKV_EXTRA_HIPCC_FLAGS, for builds of the tuning variants
    (e.g. -DPKV_MFMA_MIN_GROUP_D64=9 -DPKV_MFMA_MIN_GROUP_D128=9: the VALU first pass for
    every group size)."""
    return os.environ.get("PKV_EXTRA_HIPCC_FLAGS", "").split()


def _hip_flags():
    # -amdgpu-mfma-vgpr-form: matrix-core accumulators in ordinary VGPRs rather than AGPRs.
    # The prefill's softmax rescales its accumulators on the VALU, which cannot read AGPRs:
    # with them in AGPRs every block copied 32 of them out and back (and the kernel ran at
    # three waves per SIMD instead of four).
    return ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link libpkv.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc, *_hip_flags(), *_extra_flags(), "-c", os.path.join(CSRC, src), "-o",
                     obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-I", INCLUDE, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max(1, min(len(jobs), os.cpu_count() or 1, 16))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
