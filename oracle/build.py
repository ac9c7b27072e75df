"""Build the CPU oracle library (test infrastructure only).

Compiles ``alspec_oracle.c`` with gcc into ``liboracle.so`` next to this file.
Plain ``-O2`` with no fast-math and no FMA contraction, so every operation is
an IEEE double operation in program order.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "alspec_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L",
           "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
