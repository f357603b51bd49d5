"""Build libpagedattn.so in place with hipcc for gfx950.

Usage: ``python -m paged_kv_decode_slot_amd.build``.  The library is written
next to this file, where the binding loads it from.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("pagedattn.hip", "blockpool.hip")]
HEADER = os.path.join(ROOT, "include", "pagedattn.h")
LIB = os.path.join(PKG, "libpagedattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
