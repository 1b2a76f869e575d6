"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

bsattn.cpp (argument checks, forced-set and workspace layout, launch plans) is
compiled with host sanitizers into a library that takes the kernels' launchers
from the regular in-tree build, and the ABI tests run against it in a child
process with the sanitizer runtime preloaded; any report stops the run.  No GPU
is touched: the ABI tests only take the paths that return before a launch.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sliding_window_attention_block_amd")
LIB = os.path.join(PKG, "libbsattn.so")


def _asan_runtime():
    for pat in ("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def test_abi_under_host_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = _asan_runtime()
    if not os.path.exists(hipcc) or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not installed")
    assert os.path.exists(LIB), "build the library first (__graft_entry__.build())"
    obj = str(tmp_path / "bsattn_san.o")
    out = str(tmp_path / "libbsattn_san.so")
    # sanitizers on the host side of the compile only (there is no device code in
    # bsattn.cpp, and none is built with them)
    subprocess.run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    "-c", os.path.join(PKG, "csrc", "bsattn.cpp"), "-o", obj],
                   check=True, capture_output=True, text=True)
    subprocess.run([hipcc, "-shared", "-fPIC", obj, "-L" + PKG, "-l:libbsattn.so", "-Wl,-rpath," + PKG, "-o", out],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, LD_PRELOAD=rt, BSATTN_LIBRARY=out,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
