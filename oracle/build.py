"""Compile the fp64 CPU oracle (oracle.c) into liboracle.so with gcc.

Test infrastructure: built for the test suite, the smoke check and the
benchmark's CPU-baseline leg; the product library never links it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -O2 without fast-math: the compiler may not reorder the floating-point sums.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
          "-ffp-contract=off"]


def build(out=LIB, defines=()):
    """Compile oracle.c to `out`; `defines` are extra -D flags (the mutation
    test uses them to plant mistakes in a private copy)."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *[f"-D{d}" for d in defines], SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
