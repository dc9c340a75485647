"""Build the HIP library libmoe.so (gfx950) in-tree with hipcc."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["moe_api.hip", "route.hip", "experts.hip", "route_compare.hip", "attention.hip"]

# Packed fp32 VALU forms are disabled for all device code (they are not used
# deliberately anywhere; plain fp32 arithmetic is what the kernels mean).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-parameter",
]


def build(verbose: bool = False, extra_flags=(), out=None) -> str:
    lib = out or LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
