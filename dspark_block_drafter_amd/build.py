"""Builds libdspark.so (hipcc, gfx950) in the package directory."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libdspark.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["lmhead_gemm.hip", "lmhead_q4.hip", "markov_chain.hip", "lattice_verify.hip",
           "dspark_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off: the compiler would otherwise emit them from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source flags. The chain kernels keep their MFMA accumulators in ordinary
# VGPRs: the score of a tile starts from the logits and its top-k work reads
# the result, so accumulators in AGPRs cost a copy in and a copy out per tile
# (chain + finalize 107 -> 101 us per call at the Qwen3-8B shape, 53 -> 51 us
# at the Gemma shape, identical results).
# The 4-bit projection scales every MFMA result with VALU FMAs, so it takes
# the same form (FM = 4: 494 -> 216 registers, occupancy 1 -> 2).
SOURCE_FLAGS = {"markov_chain.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "lmhead_q4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build() -> str:
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
