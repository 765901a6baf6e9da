"""Build the HIP library ``libpmqa.so`` (and the measurement library
``libpmqa_ceiling.so``) in-tree for gfx950.

Usage: ``python paged_mqa_logits_amd/build.py`` (run as a script: importing the
package would first load the library this builds).
Every HIP translation unit is compiled with hipcc for gfx950 only, with packed
fp32 instructions disabled, then linked into one shared library next to this
file, where the Python binding loads it.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libpmqa.so")
# streaming ceiling kernels timed beside the logits call (bench.py only)
CEILING_LIB = os.path.join(HERE, "libpmqa_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
OBJDIR = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "schedule.hip", "logits_fp8.hip", "logits_fp4.hip", "tail_fill.hip",
           "append.hip", "topk.hip"]
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"]
# MFMA results go straight to VGPRs: with one wave per SIMD the register
# budget exceeds 256, where the compiler would otherwise pick the AGPR form
# and copy every accumulator back with v_accvgpr_read.
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + COMMON + (DEVICE if src.endswith(".hip") else []) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every source and link libpmqa.so and libpmqa_ceiling.so;
    returns the logits library's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
