"""Build librola.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librola.so")
SOURCES = [os.path.join(CSRC, "rola_kernels.hip"), os.path.join(CSRC, "rola_backward.hip"),
           os.path.join(CSRC, "rola_gemm.hip"), os.path.join(CSRC, "rola_noalloc.hip"),
           os.path.join(CSRC, "rola_api.cpp")]
HEADERS = [os.path.join(CSRC, "rola_internal.h"), os.path.join(CSRC, "rola_device.h"),
           os.path.join(os.path.dirname(PKG), "include", "rola.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


BUILDINFO = LIB + ".srchash"


def source_hash() -> str:
    h = hashlib.sha256()
    for p in SOURCES + HEADERS:
        with open(p, "rb") as f:
            h.update(f.read())
    # the flags without the include path, which names this checkout's
    # location: a copy of the tree elsewhere hashes the same
    h.update(" ".join(f for f in HIPCC_FLAGS if not f.startswith("-I")).encode())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    """Compile every HIP source into librola.so next to this file (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    with open(BUILDINFO, "w") as f:
        f.write(source_hash())
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB) or not os.path.exists(BUILDINFO):
        return True
    with open(BUILDINFO) as f:
        return f.read().strip() != source_hash()


def ensure_built() -> str:
    if stale():
        build()
    return LIB
