"""Builds the HIP library cache_gather_amd/libhc.so for gfx950 with hipcc, and
its test build cache_gather_amd/libhc_test.so.

Every kernel source is compiled for gfx950 only, with packed-fp32 instructions
disabled, and linked with the host orchestration into one shared library that
exports the C ABI of include/hc.h.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhc.so")
TEST_LIB = os.path.join(HERE, "libhc_test.so")
SOURCES = ["hc_ctx.hip", "k_topk.hip", "k_select.hip", "k_gather.hip", "k_ring.hip", "k_round.hip", "k_attend.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build() -> str:
    """Builds libhc.so and its test build libhc_test.so (the same sources with
    HC_TEST_HOOKS: hc_test_hook, for the tests of the failure paths); returns
    the path of libhc.so."""
    jobs = [(src, variant) for variant in ("", "_test") for src in SOURCES]

    def compile_one(job):
        src, variant = job
        out_dir = BUILD + variant
        os.makedirs(out_dir, exist_ok=True)
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        extra = ["-DHC_TEST_HOOKS"] if variant else []
        cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s%s" % (src, r.stdout, r.stderr))
        return obj

    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        objs = list(ex.map(compile_one, jobs))
    for variant, lib in (("", LIB), ("_test", TEST_LIB)):
        vobjs = [o for o in objs if os.path.dirname(o) == BUILD + variant]
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *vobjs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build())
