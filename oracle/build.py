"""Build the CPU oracle (test infrastructure) into oracle/libmxq_oracle.so.

Plain gcc, -O2, no fast-math and no floating-point contraction, so that every
double operation in the oracle is a single IEEE rounding.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mxq_oracle.c")
LIB = os.path.join(HERE, "libmxq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-fvisibility=hidden", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
