"""Build libfa.so (the attention kernels and the C ABI of include/fa.h) and
libfa_probe.so (the matrix-core rate probe of include/fa_probe.h, a
measurement aid) for gfx950 with hipcc.

Run ``python exact_io_aware_11_amd/build.py`` (as a script: importing the package
loads the library, which may not exist yet).  Each .hip source is compiled
to an object in _build/ (in parallel), then linked into the shared libraries
next to this file, where the Python binding loads them.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libfa.so")
PROBE_LIB_PATH = os.path.join(HERE, "libfa_probe.so")
SOURCES = ["fa_api.hip", "fwd_bf16.hip", "fwd_bf16_pp.hip", "fwd_bf16_w64.hip", "fwd_fp8.hip",
           "f32_kernels.hip", "bwd_bf16.hip", "std_attn.hip"]
PROBE_SOURCES = ["peak_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are switched off for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


# The forward kernels take row maxima of matrix-core results, which are never
# NaN for finite inputs; without NaN semantics fmaxf needs no quieting of its
# operands and fuses into three-input max instructions.
# In the backward kernels the score accumulators are read by vector ALU ops
# every tile; asking the compiler to keep matrix-core results in ordinary VGPRs
# (not accumulation registers) saves one register move per element.  The same
# holds for the 64-rows-per-wave forward, which needs the whole register file.
FILE_FLAGS = {"fwd_bf16.hip": ["-fno-honor-nans"], "fwd_fp8.hip": ["-fno-honor-nans"],
              "fwd_bf16_pp.hip": ["-fno-honor-nans"],
              "fwd_bf16_w64.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(path)} failed:\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
