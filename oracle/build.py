"""Compile the CPU oracle (plain C, fp64, OpenMP) into oracle/liboracle.so.

Test infrastructure: the oracle is a checker for the HIP path, never a
fallback for it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "paged_attention_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           SOURCE, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
