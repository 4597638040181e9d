"""Build the HIP libraries in-tree for gfx950.

    python -m transformer_attention_05_amd.build

libmi_attn.so is the release library; libmi_attn_debug.so is built from the
same sources with MI_ATTN_DEBUG=1 (the kernels also record malformed
device-side inputs, read back by attn_debug_flags).  Every source is compiled
(in parallel) on each call; the shared objects land next to this file, where
the Python binding loads them.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmi_attn.so")
LIB_DEBUG = os.path.join(PKG, "libmi_attn_debug.so")

SOURCES = ["prefill.hip", "decode.hip", "mixed.hip", "rope_write.hip", "copy_blocks.hip", "rmsnorm.hip", "api.cpp",
           "pool.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _flags(src: str):
    common = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
    if src.endswith(".hip"):
        # packed fp32 instructions are disabled for all device code
        # MFMA accumulators in VGPRs: the softmax works on them directly
        return common + ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
                         "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast",
                         "-mllvm", "--amdgpu-mfma-vgpr-form"]
    return common + ["-D__HIP_PLATFORM_AMD__"]


def _compile(job) -> str:
    src, debug = job
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *_flags(src), *(["-DMI_ATTN_DEBUG=1"] if debug else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile and link the release library (and, with `debug`, the debug
    library); returns the release library's path."""
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    variants = (False, True) if debug else (False,)
    jobs = [(src, d) for d in variants for src in SOURCES]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, jobs))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    if verbose:
        print(f"built {LIB}")
    if debug:
        _link(objs[n:], LIB_DEBUG)
        if verbose:
            print(f"built {LIB_DEBUG}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
