"""Compile the C++ oracle into oracle/liboracle.so with the system g++.

Plain -O2 with OpenMP and no floating-point contraction, so that every fp32
product is rounded before it is added (the sums follow the plain definition).
No -march: the library must run on any x86-64 host it is copied to.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dg_moe_oracle.cpp")
SOURCES = [SRC, os.path.join(HERE, "canvas_head_oracle.cpp")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           *SOURCES, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
