"""Builds the CPU oracle (test infrastructure) with gcc.

-O2 -fno-fast-math -ffp-contract=off: every arithmetic operator in the C
source is one correctly rounded IEEE operation; no fused multiply-add is
formed unless the source calls fma/fmaf.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lca_oracle.c")
LIB = os.path.join(HERE, "liblca_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
