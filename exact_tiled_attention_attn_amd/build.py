"""Build libattn.so (the C-ABI library) in-tree for gfx950 with hipcc.

Usage: ``python -m exact_tiled_attention_attn_amd.build [-j N]``.  Every
translation unit is compiled to ``_build/*.o`` in parallel and linked into
``exact_tiled_attention_attn_amd/libattn.so``.  Always recompiles.
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libattn.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_kv.hip", "attn_bwd_kv2.hip", "attn_bwd_dq.hip",
           "attn_bwd_dq_pipe.hip", "attn_aux.hip", "attn_scratch.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
DEVICE = [
    "--offload-arch=gfx950",
    # Never emit packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Keep MFMA sources and accumulators in VGPRs (files whose kernels fit in 256
# VGPRs: with AGPR-form MFMAs their loop-carried accumulators were copied
# between AGPRs and VGPRs every iteration).  The pipelined dK / dV and dQ
# kernels need more than 256 registers and keep their gradient accumulators
# in AGPRs.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
AGPR_FORM_SOURCES = {"attn_bwd_kv.hip", "attn_bwd_dq_pipe.hip"}


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if src.endswith(".hip"):
        form = [] if src in AGPR_FORM_SOURCES else VGPR_FORM
        cmd = [HIPCC, "-x", "hip", *DEVICE, *form, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-Wall", "-Wextra", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    if warn.strip():
        print(warn, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args()
    build(a.j)
