"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle's own pins (top-K, LRU, dequant, the whole-step model with its
threads, rounds, ring and attention) run again in a child process against
oracle.c built with -fsanitize=address,undefined, the sanitizer runtimes
preloaded; any out-of-bounds access, use after free or undefined operation
aborts the child.  Skipped where gcc has no sanitizer runtimes.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["test_oracle_topk.py", "test_oracle_lru.py", "test_oracle_dequant.py",
         "test_oracle_model.py", "test_oracle_mtp.py", "test_oracle_ring.py",
         "test_oracle_replacement.py", "test_oracle_attend.py", "test_oracle_format.py"]


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_pass_under_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not available")
    sys.path.insert(0, ROOT)
    from oracle import build as orc_build
    lib = orc_build.build(force=True, sanitize=True)
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=asan + " " + ubsan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", t) for t in TESTS]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
