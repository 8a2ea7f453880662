"""Compile the C++ oracle into oracle/liboracle.so with the system g++.

-O3 with OpenMP and no floating-point contraction, so that every fp32
product is rounded before it is added, and no reassociation (no -ffast-math),
so that every sum runs in the order the definition writes it: the optimiser
may vectorise what is elementwise but not change a result.
-march=x86-64-v3 (AVX2, FMA) rather than -march=native: the library is built in
one container and run on the GPU host's CPU, which need not be the same model;
every x86-64 server CPU of the last decade runs x86-64-v3 code.

`python -m oracle.build --sanitize` builds oracle/liboracle_san.so instead, with
AddressSanitizer and UndefinedBehaviorSanitizer (every finding fatal); the
binding loads it when DG_ORACLE_LIB names it, with the sanitizer runtimes
preloaded into the Python process (see sanitize_env()).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dg_moe_oracle.cpp")
SOURCES = [SRC, os.path.join(HERE, "canvas_head_oracle.cpp")]
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
FLAGS = ["-std=c++17", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared"]
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    opt = SAN_FLAGS if sanitize else ["-O3", "-march=x86-64-v3"]
    cmd = ["g++", *opt, *FLAGS, *SOURCES, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sanitize_env() -> dict:
    """Environment for a Python process that loads the sanitized oracle: the ASan and UBSan runtimes
    preloaded (Python itself is not instrumented), leak checks off (the interpreter keeps its memory
    until exit)."""
    rt = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True, check=True).stdout.strip()
          for n in ("libasan.so", "libubsan.so")]
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(rt)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["DG_ORACLE_LIB"] = SAN_LIB
    return env


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
