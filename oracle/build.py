"""Compile the fp64 CPU oracle into oracle/libtvoracle.so (gcc, OpenMP, -O2, no fast-math).

Test infrastructure: the library is loaded only by the tests, the smoke check
and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "libtvoracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           os.path.join(HERE, "tv_oracle.c"), "-o", SO + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
