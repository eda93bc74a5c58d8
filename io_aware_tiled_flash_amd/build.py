"""Compile the HIP sources of the attention library into ``libfa.so`` (gfx950).

Usage: ``python -m io_aware_tiled_flash_amd.build`` (or ``build()`` from
Python).  Every source is compiled on each call; objects go to ``_build/``
next to the package and the shared library is written in-tree, next to this
file, where the binding loads it.
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
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.hip", "fa_fwd_mfma.hip", "fa_fwd_f32.hip", "fa_bwd_mfma.hip", "fa_decode.hip"]
# Measurement support for the benchmark (shader-clock sampler), kept out of
# the attention library's ABI.
CLOCK_LIB = os.path.join(PKG, "libfa_clock.so")
CLOCK_SOURCES = ["fa_clock.hip"]

# Per-source extra flags for the matrix-core kernel:
#  * it never produces or consumes NaN (masked scores are -inf, which stays
#    honoured), so NaN-quieting of min/max operands is dropped;
#  * MFMA results (scores, output accumulators) are kept in VGPRs, where the
#    softmax and the rescale use them, instead of AGPRs that would need a
#    copy for every vector-ALU access.
#  The backward and decode kernels use the VGPR-destination form too: their
#  score blocks are read by the vector ALU every tile, and with AGPR results
#  each read is a copy (a third of the dQ kernel's vector work; the decode
#  matrix-core kernel ran at 2.9 TB/s that way and at 4.6 TB/s without).
EXTRA_FLAGS = {"fa_fwd_mfma.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
               "fa_bwd_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "fa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def device_asm(src: str, out: str) -> str:
    """Device assembly of one source, compiled with exactly the library's
    flags (for checks of the generated code; the library is not touched)."""
    cmd = [_hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stderr}")
    return out


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CLOCK_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CLOCK_SOURCES], CLOCK_LIB)
    if verbose:
        print(f"built {LIB} and {CLOCK_LIB}")
    return LIB


if __name__ == "__main__":
    build()
