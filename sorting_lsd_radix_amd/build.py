"""Build the gfx950 HIP library ``librs.so`` in-tree with hipcc."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "librs.so")
SOURCES = ["radix.hip", "compact.hip", "scan.hip", "bitonic.hip", "rs_api.cpp"]
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


# The same sources built with the ballot rank forced on every path (the
# library's default ranks with LDS atomics whose same-address lanes gfx950
# serves in lane order); the GPU tests run a parity subset against it.
BALLOT_LIB_PATH = os.path.join(PKG, "librs_ballot.so")
BALLOT_FLAGS = ["-DRS_FORCE_BALLOT_RANK"]


def compile_library(out, extra_flags=(), verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra_flags) + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose=False, extra_flags=(), ballot_variant=True):
    """Compile every source into librs.so (always recompiles), and the
    forced-ballot variant librs_ballot.so beside it."""
    jobs = [(LIB_PATH, list(extra_flags))]
    if ballot_variant:
        jobs.append((BALLOT_LIB_PATH, list(extra_flags) + BALLOT_FLAGS))
    if len(jobs) == 1:
        return compile_library(LIB_PATH, extra_flags, verbose)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(jobs)) as ex:
        for f in [ex.submit(compile_library, out, fl, verbose) for out, fl in jobs]:
            f.result()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
