"""Build libdgmoe.so (the HIP library behind include/dg_moe.h and include/dg_head.h) for gfx950 with hipcc.

Usage: python -m expert_ffn_canvas_amd.build   (or build() from Python)
Each source is compiled to an object in parallel (no device code crosses a file), then the objects are
linked into the library next to this file; every call recompiles.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdgmoe.so")
SOURCES = ["dg_moe_host.hip", "router.hip", "permute.hip", "gemm_bf16.hip", "gemm_i4.hip", "gemm_q8.hip",
           "gemm_mx.hip", "combine.hip", "head.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions stay off (plain fp32 code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-variable",
]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    return res.returncode, err


def build(verbose: bool = False, extra_flags=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="dgmoe_build_") as tmpdir:
        jobs = []
        for s in SOURCES:
            obj = os.path.join(tmpdir, os.path.splitext(s)[0] + ".o")
            jobs.append((obj, [hipcc, *HIPCC_FLAGS, *extra_flags, *inc, "-c", os.path.join(CSRC, s), "-o", obj]))
        if verbose:
            for _, cmd in jobs:
                print(" ".join(cmd), flush=True)
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(workers) as pool:
            results = list(pool.map(lambda j: _run(j[1]), jobs))
        for (obj, cmd), (rc, err) in zip(jobs, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
        tmp = LIB + ".tmp"
        link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
