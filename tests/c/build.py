"""Builds tests/c/sl_c_roundtrip, the C host program the C-boundary GPU test
runs (gcc, C99, linked against libsparseloco.so and the HIP runtime)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "sl_c_roundtrip.c")
EXE = os.path.join(HERE, "sl_c_roundtrip")
PKG = os.path.join(ROOT, "communication_efficient_distributed_amd")
ROCM = "/opt/rocm"


def build_c_roundtrip(out: str = EXE, verbose: bool = False) -> str:
    """Compile the program to `out`; the library is found next to the package
    through an rpath relative to `out` when `out` is the default location."""
    rpath_pkg = "$ORIGIN/../../communication_efficient_distributed_amd" if out == EXE else PKG
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-L", PKG, "-lsparseloco", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{rpath_pkg}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_c_roundtrip(verbose=True))
