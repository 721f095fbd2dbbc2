"""Build the CPU oracle (test infrastructure only) with gcc.

    python oracle/build.py        -> oracle/liboracle.so

The oracle is plain C99 + OpenMP, compiled for the host.  It is built beside
the HIP library so that the tests and the benchmark's CPU-baseline leg can
load it; nothing in the product path links it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Werror", *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
