"""Build libw4.so (gfx950) in-tree with hipcc.

    python weight_only_bit_unpack_amd/build.py

Every source under csrc/ is compiled for gfx950 only; the objects go to
csrc/_build/ and the shared library to this package directory, where the
binding loads it from.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libw4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["w4_api.cpp", "w4_quantize.hip", "w4_dequant.hip", "w4_gemv.hip", "w4_gemm.hip",
           "w4_workspace.cpp", "w4_fit.hip", "w4_noalloc.hip"]

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE arithmetic: no contraction of separate multiplies and adds
    "-ffp-contract=off",
    # keep packed-fp32 instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _compile(src):
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


# Measurement context for the benchmark only (a plain streaming read); its
# own library so that nothing of it is in libw4.
CTX_SOURCES = ["ctx_read.hip"]
CTX_LIB = os.path.join(PKG, "libw4ctx.so")


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(CTX_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + CTX_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CTX_LIB)
    if verbose:
        print(f"built {LIB} and {CTX_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
