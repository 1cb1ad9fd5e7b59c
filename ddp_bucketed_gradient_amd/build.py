"""Build the native libraries in-tree.

* ``lib/libddpb.so``           -- the product: host core + C ABI + gfx950 kernels,
                                  compiled by hipcc.
* ``lib/libddpb_hostonly.so``  -- test build of the same host core and C ABI
                                  with a launcher that enqueues nothing, compiled
                                  by g++; lets CPU-only tests drive the planner
                                  and the readiness state machine. It never
                                  touches gradient data, and the Python binding
                                  only loads it when a test asks for it by name.

Usage: ``python -m ddp_bucketed_gradient_amd.build [--hip-only|--host-only]``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
HIP_LIB = os.path.join(LIBDIR, "libddpb.so")
HOST_LIB = os.path.join(LIBDIR, "libddpb_hostonly.so")
ARCH = "gfx950"

HOST_SOURCES = ["plan.cpp", "core.cpp", "abi.cpp"]

# -ffp-contract=off: no fused multiply-add may change the rounding of the mean.
# packed-fp32-ops disabled: the float4 adds stay scalar v_add_f32.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               "-ffp-contract=off", "-fno-fast-math",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; install ROCm or set HIPCC")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_hip(out: str = HIP_LIB) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES + ["kernels.hip"]]
    tmp = out + ".tmp"
    _run([_hipcc()] + HIPCC_FLAGS + srcs + ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-o", tmp])
    os.replace(tmp, out)
    return out


def build_hostonly(out: str = HOST_LIB) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES + ["null_launcher.cpp"]]
    tmp = out + ".tmp"
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra"] + srcs + ["-o", tmp])
    os.replace(tmp, out)
    return out


def build_all():
    build_hostonly()
    build_hip()


if __name__ == "__main__":
    args = set(sys.argv[1:])
    if "--host-only" in args:
        build_hostonly()
    elif "--hip-only" in args:
        build_hip()
    else:
        build_all()
