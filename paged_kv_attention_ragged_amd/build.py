"""Build librpa.so (the gfx950 HIP library behind include/rpa.h), in-tree.

    python -m paged_kv_attention_ragged_amd.build

Host C++ (planner, C ABI) is compiled with g++, the kernels with hipcc for
gfx950 only; the shared library lands next to this file.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librpa.so")
FLOORS_LIB = os.path.join(HERE, "librpa_floors.so")  # benchmark microkernels (bench.py only)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wall"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip", ".h")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    """Compile every source and link librpa.so (and the benchmark's
    librpa_floors.so); always rebuilds."""
    inc = ["-I", INCLUDE, "-I", CSRC]
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    tmp_floors = FLOORS_LIB + ".tmp%d" % os.getpid()
    _run([hipcc] + HIP_FLAGS + ["-shared", "-o", tmp_floors, os.path.join(CSRC, "rpa_floors.hip")], verbose)
    os.replace(tmp_floors, FLOORS_LIB)
    with tempfile.TemporaryDirectory(prefix="rpa_build_") as tmp:
        objs = []
        o = os.path.join(tmp, "rpa_schedule.o")
        _run(["g++"] + HOST_FLAGS + inc + ["-c", os.path.join(CSRC, "rpa_schedule.cpp"), "-o", o], verbose)
        objs.append(o)
        o = os.path.join(tmp, "rpa_api.o")
        _run(["g++"] + HOST_FLAGS + inc + ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
              "-c", os.path.join(CSRC, "rpa_api.cpp"), "-o", o], verbose)
        objs.append(o)
        o = os.path.join(tmp, "rpa_kernels.o")
        _run([hipcc] + HIP_FLAGS + list(extra_hip_flags) + inc +
             ["-c", os.path.join(CSRC, "rpa_kernels.hip"), "-o", o], verbose)
        objs.append(o)
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib]
             + objs + ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")],
             verbose)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
