"""Build the HIP library libmoe_vs.so in-tree for gfx950 with hipcc.

    python -m moe_variable_size_amd.build [--verbose]

Each source compiles to its own object in parallel (the files share no device
code), then hipcc links the shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_vs.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# per source: mfma.hip's weight gradient claims its next unit with an atomic
# whose result it reads only when the current unit ends; the atomic optimizer
# (one atomic per wave plus a broadcast of the result) would wait for the
# result at once
FILE_FLAGS = {"mfma.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd[-3:])}")
    if verbose and r.stderr.strip():
        # hipcc's host pass reports the device-only feature flag; keep other text
        lines = [l for l in r.stderr.splitlines()
                 if "packed-fp32-ops" not in l and "warning: feature" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")


def build(verbose: bool = False, extra=()) -> str:
    srcs = sources()
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="moe_vs_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.basename(s) + ".o") for s in srcs]
        jobs = [[HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(s), ()), *extra, *inc, "-c", "-o", o, s]
                for s, o in zip(srcs, objs)]
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            list(ex.map(lambda c: _run(c, verbose), jobs))
        tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    print(LIB)
