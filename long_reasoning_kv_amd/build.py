"""Build the HIP library ``libabk.so`` in-tree for gfx950.

``python -m long_reasoning_kv_amd.build`` compiles every source under
``csrc/`` with hipcc into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libabk.so")
SOURCES = ["csrc/abk_api.cpp", "csrc/pool.cpp", "csrc/pool_kernels.hip", "csrc/decode.hip",
           "csrc/compress.hip", "csrc/prefill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False, out: str = LIB) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp] + \
        [os.path.join(HERE, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
