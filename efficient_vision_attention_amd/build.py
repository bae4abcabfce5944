"""Builds libhsmla.so from csrc/*.hip with hipcc for gfx950.

    python -m efficient_vision_attention_amd.build

Objects go to <repo>/_build/, the library next to this file.  Every call
compiles from scratch.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhsmla.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed float32 arithmetic is switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

COMMON = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]

# Per-source code generation.  The refinement kernel rescales and reads back
# its MFMA accumulators inside its key loop; with the accumulators in
# ordinary VGPRs (instead of the accumulation registers the compiler
# otherwise picks) none of that needs register-file moves (measured: 34.2 ->
# 30.4 us on the block's refinement; the K/V kernels gained nothing).
FILE_FLAGS = {
    "k_sparse.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []),
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
