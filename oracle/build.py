"""Build the C oracle (test infrastructure only) with gcc: oracle/liboracle.so."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "recurrence.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force=True):
    """Compile recurrence.c; returns the library path.  Generic -O3 code (no
    -march=native) so the library also runs on another host's CPU."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-std=c99", "-Wall", "-shared", "-fPIC",
           "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
