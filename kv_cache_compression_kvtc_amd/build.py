"""Builds libkvtc.so in-tree: host C++ with g++, device code with hipcc for gfx950.

Run ``python -m kv_cache_compression_kvtc_amd.build`` (or call ``build()``).
Every call recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvtc.so")
ARCH = os.environ.get("KVTC_OFFLOAD_ARCH", "gfx950")

HOST_FLAGS = ["-std=c++17", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fPIC", "-Wall",
              "-I" + INCLUDE, "-I" + CSRC]
HIP_FLAGS = ["-std=c++17", "-O3", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose and (r.stdout or r.stderr):
        print(r.stdout + r.stderr, flush=True)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    host_o = os.path.join(BUILD, "kvtc_host.o")
    dev_o = os.path.join(BUILD, "kvtc_device.o")
    _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "kvtc_host.cpp"), "-o", host_o], verbose)
    _run(["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, "kvtc_device.hip"), "-o", dev_o], verbose)
    tmp = LIB + ".tmp"
    _run(["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, host_o, dev_o, "-o", tmp,
          "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
