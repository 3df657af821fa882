"""Build the hardware-property probe used by the GPU tests (test infrastructure)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblds_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build():
    tmp = LIB_PATH + ".tmp"
    subprocess.run([HIPCC, "-O2", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-o", tmp, os.path.join(HERE, "lds_lane_order.hip")], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
