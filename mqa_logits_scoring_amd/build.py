"""Build libidx_logits.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree,
and libidx_peak.so, the MFMA throughput probe bench.py reports beside it.

Usage: python -m mqa_logits_scoring_amd.build   (or build() from Python)
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libidx_logits.so")
# the matrix-core throughput probe bench.py reports beside the roofline
PEAK_LIB = os.path.join(PKG, "libidx_peak.so")
PEAK_SOURCES = ["peak.hip"]
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["api.cpp", "plan.hip", "prepare.hip", "topk.hip", "topk_fused.hip", "score_bf16.hip", "score_bf16rs.hip", "score_fp8.hip",
           "score_mxfp8.hip", "score_mxfp4.hip"]
HEADERS = ["internal.h", "score_kernel.h", "score_kernel_gh.h", "plan_segment.h", "select_wave.h", os.path.join("..", "..", "include", "idx_logits.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            # packed fp32 VALU ops stay disabled for all device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-munsafe-fp-atomics"]


# Per-source additions.  The BF16 scoring kernel runs one wave per SIMD with
# more live values than 256 VGPRs; by default the compiler then keeps the MFMA
# accumulators in AGPRs, and every epilogue read of them costs a copy to a
# VGPR.  Forcing the accumulators into VGPRs moves other values (MFMA operands,
# which can be read from AGPRs) there instead.
EXTRA_FLAGS = {"score_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "score_bf16rs.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def flags_for(src: str) -> list[str]:
    return compile_flags() + EXTRA_FLAGS.get(os.path.basename(src), [])


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *flags_for(src), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libidx_logits.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + PEAK_SOURCES))
    for lib, part in ((LIB, objs[:len(SOURCES)]), (PEAK_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *part, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


def stale() -> bool:
    """True when the library is missing or older than a source or header."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    for f in SOURCES + HEADERS:
        if os.path.getmtime(os.path.join(CSRC, f)) > t:
            return True
    return False


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
