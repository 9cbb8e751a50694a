"""Build the HIP library (libq4adamw.so) for gfx950, in-tree, and beside it
the self-test library of its exact primitives (libq4selftest.so, loaded only
by the tests) and the bandwidth probes (libq4probe.so, loaded by the
benchmark and the tests).

hipcc flags: -ffp-contract=off (no FMA contraction, so every FP32 operation
rounds where it is written); HIP's default IEEE division and square root;
packed FP32 instructions disabled at the target-feature level.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libq4adamw.so")
SOURCES = [os.path.join(CSRC, "q4_kernels.hip"), os.path.join(CSRC, "q4_abi.cpp")]
DEPS = SOURCES + [os.path.join(CSRC, "q4_internal.h"), os.path.join(CSRC, "q4_exact.h"),
                  os.path.join(CSRC, "q4_quant.h"), os.path.join(CSRC, "q4_codebooks.inc"),
                  os.path.join(ROOT, "include", "q4adamw.h")]
PROBE_PATH = os.path.join(BUILD_DIR, "libq4probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "q4_probe.hip")]
PROBE_DEPS = PROBE_SOURCES + [os.path.join(ROOT, "include", "q4probe.h")]
SELFTEST_PATH = os.path.join(BUILD_DIR, "libq4selftest.so")
SELFTEST_SOURCES = [os.path.join(CSRC, "q4_selftest.hip")]
SELFTEST_DEPS = SELFTEST_SOURCES + [os.path.join(CSRC, "q4_exact.h"), os.path.join(CSRC, "q4_quant.h"),
                                    os.path.join(CSRC, "q4_codebooks.inc")]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the GPU library cannot be built")


def _build_one(path: str, sources: list, deps: list, force: bool, verbose: bool) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    if not force and os.path.exists(path):
        t = os.path.getmtime(path)
        if all(os.path.getmtime(d) <= t for d in deps):
            return path
    tmp = path + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, path)
    return path


def build(force: bool = True, verbose: bool = False) -> str:
    """Builds the three libraries; returns the optimizer library's path."""
    _build_one(SELFTEST_PATH, SELFTEST_SOURCES, SELFTEST_DEPS, force, verbose)
    _build_one(PROBE_PATH, PROBE_SOURCES, PROBE_DEPS, force, verbose)
    return _build_one(LIB_PATH, SOURCES, DEPS, force, verbose)


if __name__ == "__main__":
    print(build(force=True, verbose=True))
