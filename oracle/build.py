"""Build step for the CPU oracle (test infrastructure only).

Compiles oracle.cpp into oracle/liboracle.so with plain g++: no fast-math, no
floating-point contraction, so every operation is the IEEE operation written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.cpp")
    tmp = LIB + ".tmp"
    cmd = [
        "g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", tmp, src,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
