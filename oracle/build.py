"""Build the CPU oracle (oracle.c -> liboracle.so) with gcc.

Test infrastructure: the oracle is loaded only by the tests, by
``__graft_entry__.smoke()`` and by the cpu_baseline leg of ``bench.py``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add may merge two roundings.
# No -ffast-math: IEEE semantics, no flush-to-zero of subnormals.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
