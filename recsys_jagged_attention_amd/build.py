"""Build libjagged_attn.so for gfx950 with hipcc (in-tree, next to this file).

Every source is compiled for gfx950 only, with packed-FP32 VALU instructions
disabled, then linked into one shared library with a plain C ABI
(include/jagged_attn.h).  Usage: python -m recsys_jagged_attention_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libjagged_attn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["ja_plan.hip", "ja_attn_mfma.hip", "ja_attn_pp.hip", "ja_attn_f32.hip", "ja_mx_quant.hip", "ja_attn_bwd.hip", "ja_attn_bwd_mfma.hip", "ja_noalloc.hip", "ja_api.cpp"]

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

# Per-source flags.  The dK/dV kernel keeps 128 fp32 accumulators per lane
# across its query loop: with the MFMAs in their AGPR form the register
# allocator moved them between AGPRs and VGPRs at every query step (about 600
# v_accvgpr moves per 32 MFMAs, which made the kernel VALU-bound); the VGPR
# form keeps everything in the 256 VGPRs, with no moves and no spills.
EXTRA = {"ja_attn_bwd_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
