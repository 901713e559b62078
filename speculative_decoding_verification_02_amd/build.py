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


if __name__ == "__main__":
    print(build(verbose=True))
