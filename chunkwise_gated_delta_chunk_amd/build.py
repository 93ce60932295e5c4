"""Build liblinattn.so (the C-ABI library) for gfx950 with hipcc, in-tree."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblinattn.so")
SOURCES = ["meta.hip", "chunk_map.hip", "chunk_reduce.hip", "chunk_reduce16.hip", "chunk_combine.hip",
           "recurrent.hip",
           "short_conv.hip", "chunk_bwd.hip", "chunk_bwd_kda.hip",
           "linattn.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # private arrays stay in registers or scratch, never in LDS: the kernels
    # size their LDS themselves
    "-mllvm", "-disable-promote-alloca-to-lds",
    # MFMA accumulators in ordinary VGPRs: the kernels scale and convert their
    # accumulators with VALU instructions, which cannot read AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    """Compile every source and link liblinattn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
