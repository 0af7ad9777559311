"""Build step for libsparseloco.so (hipcc, gfx950 only).

Every translation unit is compiled for the device with:
  -ffp-contract=off            no fused operations beyond the explicit fma
  -fhip-fp32-correctly-rounded-divide-sqrt
                               IEEE division for s/3 and theta - out/N
  -fno-gpu-flush-denormals-to-zero
                               denormals are kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                               no packed-fp32 instructions
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsparseloco.so")
ARCH = "gfx950"

SOURCES = ["sparseloco.cpp", "compress.hip", "aggregate.hip", "validate.hip"]

DEVICE_FLAGS = [
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def build_library(verbose: bool = False, extra_flags=None) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", *DEVICE_FLAGS, *(extra_flags or []),
           "-I", INCLUDE, "-I", CSRC, "-x", "hip",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True, extra_flags=sys.argv[1:]))
