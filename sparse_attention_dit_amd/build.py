"""Build step: compile the HIP sources into the in-tree shared library ``libbasa.so``.

Run ``python -m sparse_attention_dit_amd.build`` (or ``__graft_entry__.build()``).
hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbasa.so")
SOURCES = ("basa_abi.cpp", "attn_kernels.hip")
# files whose contents decide the kernels' machine code (the attention and index kernels)
KERNEL_SOURCES = ("attn_kernels.hip", "index_map.hpp", "attn_launch.hpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def kernel_hash() -> str:
    """Short digest of the kernel sources: counter summaries record it, so a summary taken
    on other kernel code is recognised as stale."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(CSRC, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    objs = []
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
              "-Wall", "-Wno-unused-command-line-argument"]
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".o")
        lang = ["-x", "hip"]
        cmd = [HIPCC, *common, *lang, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
