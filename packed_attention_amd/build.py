"""Build libmf.so for gfx950 in-tree (packed_attention_amd/libmf.so).

    python -m packed_attention_amd.build          # or packed_attention_amd.build.build()

HIP sources are compiled with hipcc for gfx950 only, with packed-fp32
instruction selection disabled; the host-only table builder is plain C++
(g++).  Objects go to packed_attention_amd/_build/, compiled in parallel.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmf.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the softmax reads the score tiles
    # with VALU instructions, which cannot take AGPR operands
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE]

# per-file additions: the attention forward's row maxima use fmaxf, which
# otherwise quiets NaN inputs with an extra instruction per operand
HIP_EXTRA = {"varlen_attn_fwd.hip": ["-fno-honor-nans"]}

HIP_SOURCES = ["abi.cpp", "modulate_rope.hip", "gated_residual.hip", "varlen_attn_fwd.hip",
               "varlen_attn_bwd.hip", "elementwise_bwd.hip",
               "block_gemm.hip", "cfg_sampler.hip", "text_encoder.hip"]
HOST_SOURCES = ["pack_tables.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libmf.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *HIP_EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
