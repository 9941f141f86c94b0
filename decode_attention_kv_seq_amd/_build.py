"""Build libattn_decode.so (the C-ABI library) for gfx950 with hipcc.

The code object is compiled ahead of time and embedded in the shared
library; nothing is compiled at run time.  Packed-FP32 instruction selection
is disabled for the whole translation unit.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "attn_decode.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_decode.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
