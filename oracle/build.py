"""Build the CPU oracle (oracle/oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure only: the oracle is the CPU reference that tests, the
smoke check and the bench's CPU-baseline leg compare against.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off keeps every fp32/fp64 operation a separately rounded IEEE
# operation (no fused multiply-add); -ffast-math is never used.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build(force=True, verbose=False):
    """Compile the oracle; with force=False only when the library is missing."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(force=True, verbose=True)
    sys.exit(0)
