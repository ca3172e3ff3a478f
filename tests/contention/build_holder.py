"""Builds tests/contention/libholder.so, the CU-holding kernel of the contention test (test
infrastructure). Called by the package build step; the GPU test only loads the result."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libholder.so")


def build():
    subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    os.path.join(HERE, "holder.hip"), "-o", LIB], check=True, capture_output=True)
    return LIB


if __name__ == "__main__":
    print(build())
