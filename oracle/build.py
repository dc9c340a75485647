"""Compile the plain C++ oracles (the layer, and the attention ops next to it)
into oracle/libmoe_oracle.so (test infrastructure).

-ffp-contract=off keeps every fp32 operation exactly as written (no fused
multiply-add), and no -ffast-math: the oracle's arithmetic is IEEE as stated.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "moe_oracle.cpp"), os.path.join(HERE, "attn_oracle.cpp")]
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
