"""Builds the C part of the oracle (test infrastructure only) with gcc.

The library lands next to its source as ``oracle/liboracle_gdn.so``.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "token_recurrence.c")
LIB = os.path.join(HERE, "liboracle_gdn.so")


def build(force: bool = True) -> str:
    """Compile ``token_recurrence.c`` into ``liboracle_gdn.so`` and return its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
