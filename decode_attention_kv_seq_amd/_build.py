"""Build libattn_decode.so (the C-ABI library) for gfx950 with hipcc.

The code objects are compiled ahead of time and embedded in the shared
library; nothing is compiled at run time.  Packed-FP32 instruction selection
is disabled for every translation unit.  The translation units are compiled
in parallel and linked into one library.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("attn_decode.hip", "attn_softmax.hip", "attn_table.hip",
                                           "attn_status.cpp")]
SRC = SOURCES[0]   # the decode kernels (their hash keys the committed counter profiles)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_decode.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _errors(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if NOISE not in l)


def build(verbose: bool = False) -> str:
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.basename(src) + ".o")
        cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", "-I", INCLUDE, "-I", CSRC, src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    failed = []
    for src, p in zip(SOURCES, procs):
        _, err = p.communicate()
        if p.returncode != 0:
            failed.append("%s:\n%s" % (os.path.basename(src), _errors(err)))
        elif verbose and _errors(err).strip():
            print(_errors(err), file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + _errors(res.stderr))
    for obj in objs:
        os.remove(obj)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
