"""Build the fp64 CPU oracle into oracle/liboq_oracle.so (gcc, -O2, OpenMP).

Test infrastructure only: the product package never builds, loads or calls
this.  No fast-math: the oracle's arithmetic must stay IEEE double.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oq_oracle.c")
OUT = os.path.join(HERE, "liboq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
           SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
