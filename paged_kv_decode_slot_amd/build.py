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
SRCS = [os.path.join(PKG, "csrc", f) for f in ("pagedattn.hip", "blockpool.hip", "rmsnorm.hip", "probe.hip")]
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


def _run(cmds, verbose):
    """Run the commands in parallel; raise with the compiler's messages if one fails."""
    noise = "is not a recognized feature for this target"
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    failed = []
    for p in procs:
        out, _ = p.communicate()
        msgs = [ln for ln in out.splitlines() if noise not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append("\n".join(msgs))
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))


def build(verbose: bool = False) -> str:
    """Compile each source to an object (in parallel), then link the shared library."""
    objs = [LIB + "." + os.path.splitext(os.path.basename(src))[0] + ".o" for src in SRCS]
    inc = ["-I", os.path.join(ROOT, "include")]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    _run([[HIPCC, *compile_flags, *inc, "-c", "-o", obj, src] for src, obj in zip(SRCS, objs)], verbose)
    tmp = LIB + ".tmp"
    _run([[HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]], verbose)
    for obj in objs:
        os.remove(obj)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
