"""Builds tests/c_abi/c_abi_check: the C-ABI check program (test infrastructure), linked against
the in-tree libqf8.so and the C oracle. Called by the package build step; the GPU test only runs
the result."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "mx_block_scaled_amax_amd")
EXE = os.path.join(HERE, "c_abi_check")


def build():
    obj = os.path.join(HERE, "qf8_oracle_c_abi.o")
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-c",
                    os.path.join(ROOT, "oracle", "qf8_oracle.c"), "-o", obj], check=True)
    main_obj = os.path.join(HERE, "c_abi_check.o")
    subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fPIE", "-c",
                    os.path.join(HERE, "c_abi_check.cpp"), "-o", main_obj], check=True)
    subprocess.run(["g++", main_obj, obj, "-L" + PKG, "-lqf8", "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,$ORIGIN/../../mx_block_scaled_amax_amd", "-Wl,-rpath,/opt/rocm/lib", "-lm",
                    "-o", EXE], check=True)
    return EXE


if __name__ == "__main__":
    print(build())
