"""bench.py's command-line contract on a host without a GPU: more than one
GPU is refused with a message before anything touches a device, and the
workload and storage options parse."""
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
    assert "one GPU" in r.stderr


def test_options_parse():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--kv-format", "--shared-kv", "--pipeline", "--layers",
                "stack_decode_1m", "pair_prefill_128k"):
        assert opt in r.stdout


def test_unknown_workload_is_rejected():
    r = run("--workload", "no_such_workload")
    assert r.returncode != 0
