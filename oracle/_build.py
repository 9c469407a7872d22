"""Build step for the CPU oracle (test infrastructure): compiles oracle.c into liboracle.so.

Plain gcc, -O2 with floating-point contraction off and no fast-math, so the library performs
exactly the IEEE operations its source writes.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build(cc: str = "gcc", extra=()) -> str:
    """Compile the oracle; returns the path of the shared library."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, *CFLAGS, *extra, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
