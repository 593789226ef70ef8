"""Build the CPU oracle (oracle/liboracle.so) with gcc.

Test infrastructure: the oracle is compiled as plain C, separately from the
HIP library, with no FMA contraction and no fast-math so that every float
operation is one IEEE-754 binary32 operation in the order the source writes.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fno-strict-aliasing", "-Wall", "-Wextra", "-Werror",
          "-shared", "-fPIC"]


def build(force=True):
    """Compile oracle.c into liboracle.so; returns the library path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
