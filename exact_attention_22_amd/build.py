"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function"]


def build(out=LIB, extra=(), verbose=False):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = out + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
