"""Build the HIP library of the MoE layer path for gfx950 (in-tree shared object).

    python -m routing_permute_grouped_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["moe_capi.hip", "route.hip", "permute.hip", "grouped_gemm.hip", "combine.hip",
           "quantize.hip", "decode_gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        return _run([HIPCC, *FLAGS, "-c", src, "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
        logs = list(pool.map(compile_one, range(len(SOURCES))))
    tmp = LIB_PATH + ".tmp"
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB_PATH)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
