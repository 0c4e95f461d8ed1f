"""Compile the CPU oracle (plain C) into oracle/liboracle.so.

Test infrastructure: the product library never links or loads this.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off keeps every multiply and add separately rounded, and no
# fast-math keeps the sequential summation order of the plain definition.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(out: str = LIB, src: str = SRC, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:]))
