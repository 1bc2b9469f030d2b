"""Build libdsa.so in-tree with hipcc for gfx950 (cross-compiles without a GPU).

    python -m sparse_attention_06_amd.build          # or sparse_attention_06_amd.build.build()
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["dsa_abi.hip", "indexer.hip", "topk.hip", "mla.hip", "mha.hip", "cache.hip", "proj.hip"]

# Packed fp32 arithmetic is disabled for all device code (a target feature, device pass only).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# The indexer kernels keep their small MFMA accumulators in VGPRs, next to the VALU epilogue that
# reads them (the attention kernel needs AGPRs for its output accumulators).
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "not a recognized feature for this target" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(jobs: int = 4) -> str:
    """Compile every HIP source and link libdsa.so; always recompiles."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


PRECISION_SRC = os.path.join(ROOT, "tests", "precision", "fp8_mfma_precision.hip")
PRECISION_BIN = os.path.join(ROOT, "tests", "precision", "fp8_mfma_precision.bin")


def build_precision_check() -> str:
    """The test program that measures the matrix cores' FP8 and f16 dot-product error (a test
    input, not part of the library)."""
    cmd = [HIPCC, "-O2", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", PRECISION_SRC, "-o", PRECISION_BIN + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the FP8 precision check:\n" + r.stdout + r.stderr)
    os.replace(PRECISION_BIN + ".tmp", PRECISION_BIN)
    return PRECISION_BIN


if __name__ == "__main__":
    print(build())
