"""Compile libdlmverify.so for gfx950 with hipcc (in-tree, next to this file)."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdlmverify.so")
SOURCES = ["api.cpp", "verify.hip", "rules.hip", "tree.hip", "attn.hip", "dual_view.hip", "noalloc.hip"]
BUILD_DIR = os.path.join(HERE, "_build")

# gfx950 only; packed fp32 arithmetic is switched off for the device code and
# floating-point contraction is off so that every fused multiply-add in the
# kernels is an explicit one (the argmax refinement recomputes scores and must
# reproduce them bit for bit).
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# The verification and dual-view kernels take finite inputs only (documented in
# the header), so their device code may assume no NaN: max() then needs no
# quieting of its operands.
PER_SOURCE_FLAGS = {
    "verify.hip": ["-Xarch_device", "-fno-honor-nans"],
    "dual_view.hip": ["-Xarch_device", "-fno-honor-nans"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdlmverify)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile the library; returns its path. Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.rsplit(".", 1)[0] + ".o")
        _run([cc, *HIPCC_FLAGS, *PER_SOURCE_FLAGS.get(src, []), *extra_flags, "-I", os.path.join(ROOT, "include"),
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
