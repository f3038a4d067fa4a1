"""Build the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so with gcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cgqa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # -O2 without -ffast-math: every sum keeps the order the loops state.
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-pthread", "-fPIC", "-shared",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
