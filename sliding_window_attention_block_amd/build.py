"""Build libbsattn.so in-tree with hipcc for gfx950.

Usage: python -m sliding_window_attention_block_amd.build [--jobs N]

Each source is compiled to an object in ``_build/`` (in parallel), then linked
into ``sliding_window_attention_block_amd/libbsattn.so``.  Always rebuilds.
"""

from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsattn.so")

# (source, extra flags): the VALU scorer is compiled once per head dimension and
# query dtype, so its many instantiations build in parallel
SOURCES = [("bsattn.cpp", ()), ("summaries.hip", ()), ("select.hip", ()), ("decode.hip", ()),
           ("prefill.hip", ()), ("probe.hip", ())] + [
    ("select_valu.hip", (f"-DBSATTN_VALU_D={d}", f"-DBSATTN_VALU_BF16={bf}")) for d in (64, 128) for bf in (0, 1)]
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _object(src, flags):
    tag = "".join("_" + f.split("=")[1] for f in flags)
    return os.path.join(BUILD, os.path.basename(src) + tag + ".o")


def _compile(item):
    src, flags = item
    obj = _object(src, flags)
    cmd = [hipcc(), *CFLAGS, *flags, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs=None, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs)
    sys.exit(0)
