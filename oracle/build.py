"""Compile the fp64 CPU oracle (test infrastructure only) into a shared library.

Plain g++ with OpenMP; no fast-math and no contraction into fused
multiply-adds, so every floating-point operation is the one written in
gdn_oracle.cpp, in the order written there.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_gdn.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "g++", "-std=c++17", "-O3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
        "-Wall", "-Wextra",
        os.path.join(HERE, "gdn_oracle.cpp"),
        "-o", LIB + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
