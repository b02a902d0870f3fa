"""Builds liboracle.so from oracle.c with the host C compiler (no HIP).

Test infrastructure only: the product library is built elsewhere and never
links this one.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(src=None, out=None, extra_flags=()):
    """Compile `src` (default oracle.c) into the shared library `out`."""
    src = src or os.path.join(HERE, "oracle.c")
    out = out or LIB
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-I", HERE, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
