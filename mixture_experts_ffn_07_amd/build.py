"""Build the HIP library libmoe_ffn.so in-tree for gfx950 with hipcc.

Every source is compiled to an object of its own, several at a time, and the
objects are linked into the shared library.  Each call compiles everything
again.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_ffn.so")
OBJ_DIR = os.path.join(os.path.dirname(PKG), "_build")
SOURCES = ["moe_ffn.cpp", "router.hip", "permute.hip", "expert_gemm.hip", "expert_gemv.hip", "decode.hip",
           "expert_valu.hip", "combine.hip", "norm.hip", "expert_mx6.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: hipcc must not form packed fp32 VALU ops on its own.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# the host pass does not know the packed-fp32 feature and says so: harmless
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in res.stderr.splitlines() if NOISE not in line)
    return res.returncode, err


def build(verbose: bool = True, jobs: int = 0) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    objs = [os.path.join(OBJ_DIR, s + ".o") for s in SOURCES]
    cmds = [[HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    if verbose:
        print(f"{HIPCC} {' '.join(FLAGS)} -x hip -c <source> ({len(SOURCES)} sources, {jobs} at a time)", flush=True)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(_run, cmds))
    for src, (rc, err) in zip(SOURCES, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build()
