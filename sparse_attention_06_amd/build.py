"""Build libdsa.so (HIP kernels + C ABI) in-tree for gfx950.

    python -m sparse_attention_06_amd.build          # or build() from Python

Compiles every source under csrc/ with hipcc into _build/ and links
sparse_attention_06_amd/libdsa.so. Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdsa.so")
BUILD = os.path.join(PKG, "_build")
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# packed-fp32 instructions stay disabled: hipcc must not form v_pk_*_f32
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
# Per-file extras. NaN inputs are outside the library's contract, so the
# indexer's ReLU (a float max) needs no IEEE NaN canonicalisation; in the
# attention kernels the same flags cost registers, so they stay off there.
# The indexer also keeps its MFMA accumulators in architectural VGPRs (its
# register budget allows it), so its epilogue needs no v_accvgpr_read moves;
# the attention kernels already get that form from the compiler.
EXTRA = {"indexer.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form"],
         "indexer_fp8.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
