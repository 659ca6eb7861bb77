"""Build liblt.so in-tree for gfx950.

    python -m weight_dequantization_amd.build

The device code is compiled for gfx950 only, with packed-fp32 instruction
selection disabled; the host packer is plain C++17.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"),
]


DEBUG_LIB = os.path.join(PKG, "liblt_debug.so")


def build(verbose: bool = False, debug: bool = True) -> str:
    """Build liblt.so and, with debug, liblt_debug.so: the same library with
    LT_DEBUG, whose decoder checks that every exec-narrowing LDS store is
    called wave-uniformly (lt_debug_violations)."""
    os.makedirs(BUILD, exist_ok=True)
    pack_o = os.path.join(BUILD, "lt_pack.o")
    api_o = os.path.join(BUILD, "lt_api.o")
    dbg_o = os.path.join(BUILD, "lt_api_debug.o")
    cmds = [
        ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-pthread", "-I" + os.path.join(ROOT, "include"), "-c",
         os.path.join(CSRC, "lt_pack.cpp"), "-o", pack_o],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "lt_api.hip"), "-o", api_o],
        [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_o, pack_o, "-pthread",
         "-o", LIB + ".tmp"],
    ]
    if debug:
        cmds += [
            [HIPCC, *HIP_FLAGS, "-DLT_DEBUG", "-c", os.path.join(CSRC, "lt_api.hip"), "-o", dbg_o],
            [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", dbg_o, pack_o, "-pthread",
             "-o", DEBUG_LIB + ".tmp"],
        ]
    for c in cmds:
        if verbose:
            print(" ".join(c), flush=True)
        r = subprocess.run(c, capture_output=True, text=True)
        err = "\n".join(l for l in (r.stderr or "").splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("build step failed: %s\n%s" % (" ".join(c), err))
        if verbose and err.strip():
            print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    if debug:
        os.replace(DEBUG_LIB + ".tmp", DEBUG_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
