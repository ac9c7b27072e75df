"""Build libalspec_synth.so: the device half of the input generator and the
bandwidth probes the benchmark uses."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "synth_kernels.hip"),
        os.path.join(HERE, "probe_kernels.hip")]
LIB = os.path.join(HERE, "libalspec_synth.so")


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", LIB + ".tmp"] + SRCS
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
