"""Builds the CPU oracle (plain C, gcc) into oracle/liborc.so.

Test infrastructure only: the oracle is built so that tests, the smoke check
and the benchmark's CPU-baseline leg can call it; the product never links it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liborc.so")
# The same source built with AddressSanitizer and UndefinedBehaviorSanitizer,
# for checking the oracle itself (load it through ORACLE_LIB with the
# sanitizer runtimes preloaded).
LIB_SANITIZED = os.path.join(HERE, "liborc_sanitized.so")


def build(force: bool = True, sanitize: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    lib = LIB_SANITIZED if sanitize else LIB
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(src):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["gcc", "-std=c11", *opt, "-fPIC", "-shared", "-Wall", "-Wextra",
           "-D_GNU_SOURCE", "-o", tmp, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build())
