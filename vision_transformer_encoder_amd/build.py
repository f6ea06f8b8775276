"""Build libvit.so (HIP, gfx950 only) in-tree with hipcc.

Usage: ``python -m vision_transformer_encoder_amd.build`` or ``build()``.
Every call recompiles every source (no caching): objects go to
``vision_transformer_encoder_amd/_build/``, the library to
``vision_transformer_encoder_amd/libvit.so``; the benchmark's MFMA peak probe
(csrc/peak) to ``vision_transformer_encoder_amd/libvit_peak.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvit.so")
# measurement probe of the benchmark (dense MFMA issue rate), not the tower
PEAK_SRC = os.path.join(CSRC, "peak", "mfma_peak.hip")
PEAK_LIB = os.path.join(PKG, "libvit_peak.so")

SOURCES = ["quant.hip", "rope.hip", "attention.hip", "gemm.hip", "gemm_wide.hip", "merge.hip", "preprocess.hip",
           "abi.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source additions.  attention.hip: every value its max reductions see is
# finite (masked keys carry a large finite negative score), so the NaN
# quieting that IEEE fmaxf otherwise needs before each v_max is dropped.
# gemm.hip: MFMA results stay in VGPRs; left to its heuristics the compiler
# parks the per-K-block partial sums in AGPRs, and every promotion FMA then
# needs a v_accvgpr_read first.
EXTRA = {"attention.hip": ["-fno-honor-nans"], "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
MAX_SCRATCH = 32  # bytes per lane


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # no kernel may keep arrays in scratch memory or spill in its loops: that
    # traffic goes through L2/HBM and silently costs several times the
    # kernel's time.  A few registers kept across a whole persistent loop
    # (saved once, reloaded once per work item) stay under MAX_SCRATCH.
    kern, bad = None, []
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kern = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > MAX_SCRATCH:
            bad.append(f"{kern}: {m.group(1)} B/lane")
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory: " + "; ".join(bad))
    return obj


def build(verbose: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # every symbol must resolve (a kernel whose host stub was not emitted
    # links fine and only fails at load time)
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    except OSError as e:
        raise RuntimeError(f"linked library does not load: {e}") from None
    shutil.move(tmp, LIB)
    tmp = PEAK_LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", "-x", "hip", PEAK_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAK_SRC}:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, PEAK_LIB)
    if verbose:
        print(f"built {LIB} and {PEAK_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
