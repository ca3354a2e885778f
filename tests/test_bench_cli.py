"""bench.py's command line on the CPU: more than one GPU is refused with a
JSON message and exit status 2 (the W ranks are buffers in one GPU's HBM),
and --help lists the workload choices."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_help_lists_the_workloads():
    r = run("--help")
    assert r.returncode == 0
    assert "--workload" in r.stdout and "--graph" in r.stdout and "--tail" in r.stdout
