"""Compile the CPU oracle (plain C, f64) into oracle/libkvdec_oracle.so.

Test infrastructure: the oracle is built here so the tests, the smoke check
and the benchmark's CPU-baseline leg can load it.  No product code links it.

Flags are deliberately conservative: -O2 without -ffast-math or any
vectorisation hints, so the arithmetic is the plain IEEE double sequence
written in the source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvdec_oracle.c")
LIB = os.path.join(HERE, "libkvdec_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
