"""Build libvq.so for gfx950 with hipcc (cross-compiles without a GPU).

    python -m block_quantized_gemm_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libvq.so")

SOURCES = ["verify_gemm.hip", "w4a8_gemm.hip", "fp8_prefill.hip", "h32_quant.hip", "greedy_verify.hip",
           "hbm_probe.hip", "verify_noalloc.hip", "vq_api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # fp32 division must be correctly rounded (the quantizer's codes depend on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # keep MFMA results in VGPRs: the epilogue reads them at once
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive in SGPRs, written by the command
    # processor before the first instruction (at most 16 user SGPRs: the
    # kernel-argument pointer and up to 14 argument dwords), which saves the
    # memory round trip that reading them would cost at kernel start
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


# Per-source additions (none at present).
SOURCE_FLAGS = {}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvq.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *lang, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
