"""Build the fp64 oracle shared library (plain C, gcc, OpenMP).

Test infrastructure only; the product library never links it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(src=SRC, out=LIB, extra_flags=(), quiet=False):
    """Compile ``src`` into the shared library ``out``; returns ``out``."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + r.stderr)
    if r.stderr and not quiet:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
