"""Build liblinattn.so (gfx950) in-tree with hipcc.

    python -m kernelized_sequence_mixing_amd.build [-j N]

Every source is compiled to an object under ``_build/`` (in parallel), then
linked into ``kernelized_sequence_mixing_amd/liblinattn.so``. All device code
is compiled with packed-fp32 instruction selection disabled, and with matrix-core
accumulators in ordinary VGPRs (``-amdgpu-mfma-vgpr-form``): gfx950 MFMAs read and
write either register file, and the accumulation-register form made the compiler
copy every accumulator the VALU touches (the state's bf16 image, scores, outputs)
with v_accvgpr_read/write, ~11% of the elu+1 output pass's VALU instructions.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblinattn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "chunked_elu1.hip", "chunked_ssm.hip", "chunked_favor.hip", "scan.hip", "noncausal.hip", "decode.hip",
           "featuremap.hip", "backward.hip", "noncausal_bwd.hip", "noalloc.hip",
           "softmax_attn.hip", "favor_backward.hip", "columns.hip"]

HIPCC_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form",
               f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build liblinattn.so")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args()
    build(a.j)
    sys.exit(0)
