"""Compile the float64 CPU oracle (test infrastructure only) into oracle/libss_oracle.so.

Plain gcc, no fast-math: the oracle's double arithmetic stays IEEE.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ss_oracle.c")
LIB = os.path.join(HERE, "libss_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle library; returns its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c11",
           "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
