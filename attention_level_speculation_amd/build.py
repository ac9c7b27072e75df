"""Build libalspec.so (the gfx950 HIP kernels and the C ABI) in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libalspec.so")
SOURCES = ["alspec_kernels.hip", "alspec_post.hip", "alspec_scratch.hip",
           "alspec_api.cpp", "alspec_plan.cpp"]

# Packed fp32 instructions stay off (the compiler would otherwise form them
# from plain float code).  The leading scalar kernel arguments (up to 10) are
# preloaded into scalar registers at wave launch where the firmware supports
# it (the code keeps a prologue that loads them otherwise).
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Wall", "-Wno-unused-function",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-kernarg-preload-count=10"]


def build(verbose: bool = False, extra=()) -> str:
    cmd = (["hipcc"] + HIPCC_FLAGS + list(extra) +
           ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-shared",
            "-o", LIB + ".tmp"] + [os.path.join(CSRC, s) for s in SOURCES])
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
