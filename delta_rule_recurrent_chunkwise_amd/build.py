"""Build liblinattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m delta_rule_recurrent_chunkwise_amd.build

Each .hip source is compiled to an object in parallel, then linked into one
shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "liblinattn.so")
SOURCES = ["api.hip", "decode.hip", "prefill.hip", "prefill_pipe.hip", "la_par.hip", "backward.hip", "prologue.hip",
           "segmented.hip",
           "noalloc.hip"]
# the measurement harness's MFMA peak probe, a library of its own
PROBE_PATH = os.path.join(HERE, "libpeak_probe.so")
PROBE_SOURCE = "peak_probe.hip"

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions are generated (the compiler may otherwise
    # form them from scalar float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix instructions write ordinary vector registers, so a result that
    # feeds the next product is converted in place instead of first being
    # copied out of the accumulator registers (a dependent MFMA -> convert ->
    # MFMA step measured 64 instead of 104 cycles at 16 deep)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(path)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBE_SOURCE]))
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
        print(f"built {PROBE_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)
