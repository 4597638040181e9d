"""Build the HIP library libmi_attn.so in-tree for gfx950.

    python -m transformer_attention_05_amd.build

Every source is compiled (in parallel) on each call; the shared object lands
next to this file, where the Python binding loads it.
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

SOURCES = ["prefill.hip", "decode.hip", "rope_write.hip", "copy_blocks.hip", "rmsnorm.hip", "api.cpp", "pool.cpp"]
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


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *_flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
