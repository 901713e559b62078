"""Build the verify-step HIP library for gfx950, in-tree.

    python -m speculative_decoding_verification_02_amd.build

compiles csrc/*.hip into ``libspecverify.so`` next to this file.  The
packed-fp32 feature is switched off for the device code: the compiler
otherwise forms packed fp32 add/mul/fma instructions from ordinary float code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build the verify-step library")
    return exe


def compile_command(out: str = LIB_PATH) -> list[str]:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            *srcs, "-o", out]


def build(verbose: bool = False) -> str:
    """Compile the library (always, even if a built copy exists) and return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building %s failed:\n%s\n%s" % (LIB_NAME, " ".join(cmd), res.stderr[-8000:]))
    if verbose and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def sanitized_command(out: str) -> list[str]:
    """The same library with AddressSanitizer and UndefinedBehaviorSanitizer
    on its host code only (argument checks, workspace layout, launch set-up):
    every -fsanitize= goes to the host pass (-Xarch_host), the device code is
    built as usual."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    return [hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libasan",
            *srcs, "-o", out]


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the HIP toolchain (to
    preload into a process that loads the sanitized library)."""
    pats = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not pats:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return sorted(pats)[-1]


def build_sanitized(out: str) -> str:
    """Compile the host-sanitized library to `out` and return its path."""
    cmd = sanitized_command(out)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the sanitized library failed:\n%s\n%s" % (" ".join(cmd), res.stderr[-8000:]))
    return out


if __name__ == "__main__":
    print(build(verbose=True))
