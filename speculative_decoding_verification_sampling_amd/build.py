"""Build libspecv.so in-tree with hipcc for gfx950.

    python -m speculative_decoding_verification_sampling_amd.build

Compiles every HIP source under ``csrc/`` into one shared library next to
this file.  Packed fp32 instructions are disabled for all device code
(``-packed-fp32-ops``); the host pass warns that it does not know the
feature, which is harmless.
"""

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecv.so")
ARCH = "gfx950"

FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",        # every fused multiply-add in the kernels is written explicitly
    "-Wall",
    "-Wno-unused-function",
    "-fvisibility=hidden",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: cannot build libspecv")
    return exe


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out=LIB, extra_flags=(), verbose=False):
    """Compile libspecv.so; returns its path.  Raises on compiler errors."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, cwd="/tmp")
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
