"""Build libdflash2.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Usage:  python -m block_drafting_amd.build [--verbose] [--asan]

Each .hip source compiles to an object in parallel, then the objects link
into block_drafting_amd/libdflash2.so next to this file.  Always rebuilds.

--asan builds a second copy, _build/asan/libdflash2.so, whose host code (the
C ABI's argument checks and launch set-up) is instrumented with
AddressSanitizer; the device code is built as usual.  Load it with the
clang runtime preloaded (asan_runtime()) and DFLASH2_LIBRARY pointing at it.
"""
from __future__ import annotations

import argparse
import glob
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
LIB = os.path.join(HERE, "libdflash2.so")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of every kernel; -O3, hidden symbols
# except the extern "C" API.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# host-only instrumentation: each -fsanitize= directly after -Xarch_host
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdflash2)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that an --asan build needs
    preloaded (it is not linked into a shared library)."""
    cc = hipcc()
    r = subprocess.run([cc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return path


def build(verbose: bool = False, asan: bool = False) -> str:
    cc = hipcc()
    out_dir = os.path.join(BUILD_DIR, "asan") if asan else BUILD_DIR
    lib = os.path.join(out_dir, "libdflash2.so") if asan else LIB
    flags = HIPCC_FLAGS + (ASAN_FLAGS if asan else [])
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        _run([cc, *flags, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj], verbose)

    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = lib + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + (ASAN_FLAGS if asan else [])
    _run(link + ["-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--asan", action="store_true",
                    help="host AddressSanitizer build into _build/asan (the in-tree library is untouched)")
    a = ap.parse_args(argv)
    print(build(a.verbose, a.asan))


if __name__ == "__main__":
    sys.exit(main())
