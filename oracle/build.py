"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, host only.  -fno-fast-math and -ffp-contract=off keep every
float operation a single IEEE-754 operation; OpenMP only splits rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp8_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
        "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
