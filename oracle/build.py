"""Builds the CPU oracle (plain C, gcc) into oracle/liborc.so.

Test infrastructure only: the oracle is built so that tests, the smoke check
and the benchmark's CPU-baseline leg can call it; the product never links it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liborc.so")


def build(force: bool = True) -> str:
    src = os.path.join(HERE, "oracle.c")
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(src):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-D_GNU_SOURCE", "-o", tmp, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
