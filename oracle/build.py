"""Compile the CPU oracle (plain C) into oracle/liblosa_oracle.so with gcc.

Flags keep fp32 arithmetic exactly as written: no contraction into fused
multiply-adds, no fast-math, SSE scalar math (x86-64 default).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "losa_oracle.c")
LIB = os.path.join(HERE, "liblosa_oracle.so")
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wno-unused-function"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(), file=sys.stderr)
