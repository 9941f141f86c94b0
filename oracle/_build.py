"""Build the CPU oracle shared library with the host C compiler.

Plain ``gcc -O2`` with fast-math off and no FMA contraction, so the fp64
arithmetic in the oracle keeps IEEE semantics.  Test infrastructure only.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle_attn.so")


def build(src: str = SRC, lib: str = LIB, verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", lib + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
