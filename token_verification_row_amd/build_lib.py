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


# The host side (argument validation, launch geometry, error text) built with
# AddressSanitizer and UndefinedBehaviorSanitizer, for checking the C ABI on
# the CPU. Each -fsanitize= applies to the host compilation only; the device
# code is built as usual.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SANITIZED_LIB = os.path.join(BUILD_DIR, "sanitize", "libdlmverify.so")


def asan_runtime() -> str:
    """The AddressSanitizer runtime of hipcc's clang (preloaded into an uninstrumented Python)."""
    out = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang"),
                          "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.isabs(path):
        raise RuntimeError("could not locate libclang_rt.asan-x86_64.so")
    return path


def build(verbose: bool = False, extra_flags=(), sanitize: bool = False) -> str:
    """Compile the library; returns its path. Always recompiles. With sanitize, the host code is
    instrumented and the library goes to SANITIZED_LIB (never over the product library)."""
    out_dir = os.path.dirname(SANITIZED_LIB) if sanitize else BUILD_DIR
    target = SANITIZED_LIB if sanitize else LIB
    flags = [*extra_flags, *(SANITIZE_FLAGS if sanitize else [])]
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.rsplit(".", 1)[0] + ".o")
        _run([cc, *HIPCC_FLAGS, *PER_SOURCE_FLAGS.get(src, []), *flags, "-I", os.path.join(ROOT, "include"),
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = target + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *(SANITIZE_FLAGS if sanitize else []), *objs, "-o", tmp],
         verbose)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        print(build(verbose=True, sanitize=True))
        print(f"ASAN runtime: {asan_runtime()}")
    else:
        print(build(verbose=True))
