"""Builds libgpt2.so (every HIP kernel of the GPT-2 step plus its C ABI) for gfx950.

Sources are compiled in-tree with hipcc into ``_build/`` and linked into
``_lib/libgpt2.so``.  Run ``python -m gpt_decoder_pre_amd.build``.
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libgpt2.so")

ARCH = "gfx950"
SOURCES = ["gemm.hip", "attention.hip", "layernorm.hip", "embed.hip", "xent.hip", "optim.hip", "infer.hip",
           "gpt2.cpp", "train.cpp", "infer_ctx.cpp", "probe.hip"]
# The sources of the training step are built a second time for the fp16 mode:
# IEEE half as the 16-bit operand type, in namespace gpt2k_f16, with the C ABI
# entry points prefixed f16_ (the library's own entry points hand fp16
# contexts to them).
F16_SOURCES = ["gemm.hip", "attention.hip", "layernorm.hip", "embed.hip", "xent.hip", "optim.hip", "gpt2.cpp"]
F16_FLAGS = ["-DGPT2_OPS_F16", "-Dgpt2k=gpt2k_f16"]
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgpt2.so")


def _compile(job: tuple, hipcc: str) -> str:
    src, f16 = job
    obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ("_f16" if f16 else "") + ".o")
    cmd = [hipcc, *CXXFLAGS, *(F16_FLAGS if f16 else []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    # the two GEMM builds take longest: start them first
    jobs = [("gemm.hip", False), ("gemm.hip", True)] + [(s, False) for s in SOURCES if s != "gemm.hip"] + \
        [(s, True) for s in F16_SOURCES if s != "gemm.hip"]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(j, hipcc), jobs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
