"""Build the HIP library for gfx950, in-tree.

    python -m mixture_experts_layer_amd.build

compiles csrc/*.hip into mixture_experts_layer_amd/lib/libmoe_mi355x.so with
hipcc (cross-compiles without a GPU).  Packed-FP32 instructions are disabled
for every HIP source.

The library carries the SHA-256 of the sources and flags it was built from
(moe_source_sha256()); the loader refuses a library whose stamp differs from
the sources in the tree, so a stale binary is never run.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmoe_mi355x.so")
SOURCES = ["abi.hip", "route.hip", "permute.hip", "ffn.hip", "combine.hip", "decode.hip",
           "dispatch.hip", "reshard.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def source_files():
    """Every file the library is compiled from, in a fixed order."""
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))
    return files + [os.path.join(ROOT, "include", "moe.h")]


def source_sha256():
    """SHA-256 over the sources' names and bytes and the compile flags."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    flags = [f for f in HIPCC_FLAGS if not f.startswith(os.path.sep)]
    h.update(" ".join(flags + SOURCES).encode())
    return h.hexdigest()


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    stamp = f'-DMOE_SOURCE_SHA256="{source_sha256()}"'
    cmd = [hipcc()] + HIPCC_FLAGS + [stamp] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
