"""Build libparallax.so in-tree with hipcc for gfx950.

Each HIP source is compiled to an object under ``_build/`` (in parallel),
then linked into ``transformer_attention_parallax_amd/libparallax.so``.
Usage: ``python -m transformer_attention_parallax_amd.build``.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libparallax.so")

SOURCES = ["api.hip", "decode.hip", "fwd_valu.hip", "fwd_mfma.hip", "pack.hip", "bwd_mfma.hip", "decode_gqa.hip", "stream.hip", "proj.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libparallax)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
        # keep the compiler from forming packed fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


# Per-source additions. decode_gqa.hip: matrix products in their VGPR form,
# so the loop-carried accumulators of its tile loop stay in one register
# class (in the AGPR form the compiler copied all 32 of them from AGPRs to
# VGPRs and back on every tile).
EXTRA_FLAGS = {"decode_gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), *EXTRA_FLAGS.get(src, []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libparallax.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libparallax.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
