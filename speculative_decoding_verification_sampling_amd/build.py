"""Build libspecv.so in-tree with hipcc for gfx950.

    python -m speculative_decoding_verification_sampling_amd.build

Compiles every HIP source under ``csrc/`` (in parallel, one object each)
into one shared library next to this file.  Packed fp32 instructions are disabled for all device code
(``-packed-fp32-ops``); the host pass warns that it does not know the
feature, which is harmless.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, cwd="/tmp")
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)


def build(out=LIB, extra_flags=(), verbose=False):
    """Compile libspecv.so; returns its path.  Raises on compiler errors.
    Each source is compiled to an object of its own, in parallel, and the
    objects are linked into the shared library."""
    tmp = out + ".tmp"
    objdir = tempfile.mkdtemp(prefix="specv_build_")
    try:
        cflags = [f for f in FLAGS if f != "-shared"]
        jobs = []
        for src in sources():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            jobs.append(([hipcc(), *cflags, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj], obj))
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            for f in [pool.submit(_run, cmd, verbose) for cmd, _ in jobs]:
                f.result()
        _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for _, o in jobs], "-o", tmp], verbose)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
