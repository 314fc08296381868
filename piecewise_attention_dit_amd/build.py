"""Build libpisa.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m piecewise_attention_dit_amd.build   (or call build()).
Each translation unit is compiled in parallel, then linked into
piecewise_attention_dit_amd/libpisa.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpisa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["pisa_host.cpp", "stats.hip", "indexer.hip", "attn.hip", "attn_blocks.hip", "attn_f32.hip",
           "decode.hip", "roofline.hip", "attn_pivot.hip"]
ARCH = "gfx950"
# sources whose MFMA results are consumed by VALU code right away: let the
# compiler give MFMAs VGPR destinations instead of AGPRs, which would need a
# v_accvgpr_read per result register
VGPR_MFMA = {"attn_pivot.hip"}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpisa)")


def _flags(src: str) -> list[str]:
    f = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
         "-Wall", "-Wno-unused-result"]
    if src.endswith(".hip"):
        # never let the compiler form packed fp32 arithmetic (v_pk_*_f32)
        f += ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
        if src in VGPR_MFMA:
            f += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    else:
        f += ["-x", "hip"]
    return f


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *_flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (p.stdout + p.stderr).splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
