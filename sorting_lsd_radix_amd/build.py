"""Build the gfx950 HIP library ``librs.so`` in-tree with hipcc."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "librs.so")
SOURCES = ["radix.hip", "compact.hip", "bitonic.hip", "rs_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # packed fp32 instructions stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # the fully unrolled loops of the pass kernel are unrolled by an earlier
    # pass; the later pragma check then reports them as not unrolled
    "-Wno-pass-failed",
]


def build(verbose=False, extra_flags=()):
    """Compile every source into librs.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra_flags) + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
