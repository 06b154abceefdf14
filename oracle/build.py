"""Compile the CPU oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is the checker, not part of the product.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# Plain optimisation, no fast-math and no FMA contraction: every product of
# two fp32 or fp16 values is exact in double, and the per-element sum keeps
# its k-ascending order.
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build_oracle(force=True):
    """Compile liboracle.so; returns its path.  Raises on compiler error."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle())
