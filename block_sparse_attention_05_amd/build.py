"""Build libsparse_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m block_sparse_attention_05_amd.build`` (or call ``build()``).
Each translation unit is compiled to an object in ``_build/`` in parallel,
then linked into ``block_sparse_attention_05_amd/libsparse_attn.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libsparse_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["abi.cpp", "pool.hip", "route.hip", "attn.hip", "attn_pair.hip", "spark.hip",
           "static_scratch.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


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
    return out


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (device code is compiled as usual): `python -m
# block_sparse_attention_05_amd.build --sanitize` writes it to
# _build/sanitize/libsparse_attn.so, for the host validation tests.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-g"]
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")


def build(verbose: bool = False, extra_flags=(), sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library.
    Always recompiles.  Returns the library path.  With ``sanitize`` the
    host code is built with ASan/UBSan into _build/sanitize/ instead."""
    hipcc = _hipcc()
    out_dir = SANITIZE_DIR if sanitize else BUILD_DIR
    lib_path = os.path.join(SANITIZE_DIR, LIB_NAME) if sanitize else LIB_PATH
    if sanitize:
        extra_flags = (*extra_flags, *SANITIZE_FLAGS)
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *COMMON_FLAGS, *extra_flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append(cmd)
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = lib_path + ".tmp"
    link_extra = ["-fsanitize=address", "-fsanitize=undefined"] if sanitize else []
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs], verbose)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
