"""Builds libkvtc.so in-tree: host C++ with g++, device code with hipcc for gfx950.

Run ``python -m kv_cache_compression_kvtc_amd.build`` (or call ``build()``).
Every call recompiles.  The translation units compile in parallel; the fetch
kernel is instantiated once per contraction length, each in its own unit.

The library carries the hash of the sources it was built from
(``kvtc_build_id()``); ``source_hash()`` computes the same hash of the current
tree, so a caller can tell a stale library from a current one.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
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
FETCH_KS = range(1, 17)            # fetch contraction lengths, in 16-slot k-steps

HOST_FLAGS = ["-std=c++17", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fPIC", "-Wall",
              "-I" + INCLUDE, "-I" + CSRC]
HIP_FLAGS = ["-std=c++17", "-O3", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC]


def source_files():
    """Every file the library is compiled from, in a fixed order."""
    pats = [os.path.join(CSRC, "*.cpp"), os.path.join(CSRC, "*.hip"), os.path.join(CSRC, "*.h"),
            os.path.join(INCLUDE, "*.h")]
    return sorted(f for p in pats for f in glob.glob(p))


def source_hash() -> str:
    """First 16 hex digits of the SHA-256 over the library's sources (name and bytes of each)."""
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose and (r.stdout or r.stderr):
        print(r.stdout + r.stderr, flush=True)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    bid = source_hash()
    steps = [["g++", *HOST_FLAGS, f'-DKVTC_BUILD_ID="{bid}"', "-c", os.path.join(CSRC, "kvtc_host.cpp"),
              "-o", os.path.join(BUILD, "kvtc_host.o")]]
    objs = [steps[0][-1]]
    for name in ("kvtc_device", "kvtc_append", "kvtc_append_i8", "kvtc_attend", "kvtc_refit", "kvtc_fit", "kvtc_probe", "kvtc_entropy"):
        o = os.path.join(BUILD, name + ".o")
        steps.append(["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, name + ".hip"), "-o", o])
        objs.append(o)
    for ks in FETCH_KS:
        o = os.path.join(BUILD, f"kvtc_fetch_ks{ks}.o")
        steps.append(["hipcc", *HIP_FLAGS, f"-DKVTC_FETCH_KS={ks}", "-c",
                      os.path.join(CSRC, "kvtc_fetch_ks.hip"), "-o", o])
        objs.append(o)
    jobs = jobs or min(16, os.cpu_count() or 1)
    # the slowest units first
    steps.sort(key=lambda c: 0 if "kvtc_fetch_ks.hip" in " ".join(c) else 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in steps]:
            f.result()
    tmp = LIB + ".tmp"
    _run(["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp, "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


def library_build_id(path: str = LIB):
    """The source hash a built library carries (the string behind kvtc_build_id()),
    read from the file without loading it, or None if it is absent or has none.
    (Loading it would pin that file in the process: a later load of the same
    path after a rebuild would return the stale library.)"""
    if not os.path.exists(path):
        return None
    import re
    with open(path, "rb") as fh:
        m = re.search(rb"kvtc-build-id:([0-9a-f]{16})", fh.read())
    return m.group(1).decode() if m else None


def ensure_current(verbose: bool = False, log=None) -> str:
    """Rebuild the library unless it was built from the current sources."""
    want, have = source_hash(), library_build_id()
    if have != want:
        if log:
            log(f"libkvtc.so build id {have} != source hash {want}: rebuilding")
        build(verbose=verbose)
        have = library_build_id()
        if have != want:
            raise RuntimeError(f"rebuilt libkvtc.so reports build id {have}, expected {want}")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
