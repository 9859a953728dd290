"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so with g++."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "alexnet_oracle.cpp")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = True) -> str:
    cmd = ["g++", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c++17",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
