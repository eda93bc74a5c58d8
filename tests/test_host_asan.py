"""The library's host code (argument validation, dispatch, error text) under
AddressSanitizer, on the CPU.

fa_api.hip is recompiled with AddressSanitizer on its host side only, linked
with the already-built kernel objects into a separate library, and the host
boundary tests (tests/test_boundary.py, which launch nothing) run against it
in a child process with the sanitizer runtime preloaded.  Any out-of-bounds
access, use after free or similar in the validation code fails this test.
No GPU is involved.
"""
import os
import subprocess
import sys

import pytest

from io_aware_tiled_flash_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_DIR = os.path.join(B.BUILD, "asan")
# host side only: device code is never built with a sanitizer here
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    r = subprocess.run([B._hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isfile(path):
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    return path


@pytest.fixture(scope="module")
def asan_library():
    kernels = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o")
               for s in B.SOURCES if s != "fa_api.hip"]
    if not all(os.path.exists(o) for o in kernels):
        B.build(verbose=False)
    os.makedirs(ASAN_DIR, exist_ok=True)
    obj = os.path.join(ASAN_DIR, "fa_api.o")
    lib = os.path.join(ASAN_DIR, "libfa_asan.so")
    cmd = [B._hipcc(), *B.HIPCC_FLAGS, "-O1", "-g", *HOST_ASAN, "-c",
           os.path.join(B.CSRC, "fa_api.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    cmd = [B._hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libasan",
           *HOST_ASAN, obj, *kernels, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return lib


def _env(lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["IO_AWARE_FA_LIBRARY"] = lib
    return env


def test_sanitizer_runtime_is_active(asan_library):
    code = ("import ctypes, io_aware_tiled_flash_amd as fa; "
            "ctypes.CDLL(None).__asan_address_is_poisoned; "
            "assert fa.library_path().endswith('libfa_asan.so'); "
            "assert fa.fa_abi_version() == 1; print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(asan_library),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]


def test_boundary_checks_under_address_sanitizer(asan_library):
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_boundary.py", "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"], cwd=ROOT,
                       env=_env(asan_library), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr
