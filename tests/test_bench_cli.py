"""bench.py's command line on the CPU: runs on several GPUs are refused with
a message and exit status 2, and the oracle baseline leg alone (--cpu-only)
prints the cpu_baseline object the GPU line carries."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_several_gpus_are_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_only_baseline_line():
    r = _bench("--cpu-only", "--workload", "tiny_4k", "--cpu-steps", "3", "--cpu-threads", "1")
    assert r.returncode == 0, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    cb = line["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "rows/s" and cb["cores"] == 1
    assert cb["value"] > 0 and "tiny_4k" in cb["sample"]
    assert line["workload"] == "tiny_4k" and line["ms_per_step"] > 0


def test_cpu_baseline_states_the_host_and_a_single_thread_rate():
    """The baseline names the host it ran on (core count, CPU model) and also
    times the oracle on one thread."""
    r = _bench("--cpu-only", "--workload", "tiny_4k", "--cpu-steps", "3", "--cpu-threads", "2",
               "--cpu-single-steps", "2")
    assert r.returncode == 0, r.stderr
    cb = json.loads(r.stdout.strip().splitlines()[-1])["cpu_baseline"]
    assert cb["cores"] == 2 and cb["nproc"] == os.cpu_count()
    assert "cpu_model" in cb
    st = cb["single_thread"]
    assert st["cores"] == 1 and st["value"] > 0 and st["unit"] == "rows/s"
