"""Build the CPU oracle (test infrastructure): oracle/libga_oracle.so.

Plain gcc, no fast-math and no FMA contraction, so every fp64 step rounds
exactly as written in ga_oracle.c.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ga_oracle.c")
LIB = os.path.join(HERE, "libga_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=gnu11", "-O2", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
