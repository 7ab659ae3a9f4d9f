"""Compile the C oracle into oracle/liboracle.so with gcc.

The oracle is plain C99 built without contraction or fast-math so that its
fp32 arithmetic is exactly the IEEE binary32 sequence written in the source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "leapq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
          "-fno-fast-math", "-fPIC", "-shared"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` to the shared object `out`; returns the output path."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
