"""Builds libevoattn.so (HIP, gfx950) in the package directory with hipcc.

Usage: python -m af3_attention_amd.build [--sanitize]

--sanitize builds libevoattn_san.so instead: the host code (argument validation,
workspace layout, dispatch) instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer against clang's shared runtime; device code is built
as usual.  It is for CPU runs of the ABI tests (tests/run_sanitizers.py).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libevoattn.so")
SAN_LIB = os.path.join(PKG, "libevoattn_san.so")

# Packed fp32 VALU instructions are disabled for all device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Host-only sanitizer flags: each -fsanitize= applies to the host pass only.
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-shared-libasan", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g",
]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    extra = SANITIZE_FLAGS if sanitize else []
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I" + INCLUDE, "-I" + CSRC, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
