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


# The same library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
# checks of the oracle itself: out-of-bounds, overflow, misaligned access).
# Loaded into an uninstrumented Python with gcc's ASan runtime preloaded.
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    flags = [f for f in CFLAGS if not (sanitize and f == "-O2")] + (SAN_FLAGS if sanitize else [])
    cmd = ["gcc", *flags, SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
