"""bench.py's command-line contract that holds without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--no-cpu"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a configuration it does not run


def test_help_lists_the_workload_switches():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0
    for opt in ("--config", "--prep", "--key-fp8", "--q-fp8", "--kv", "--score-budget", "--copy-calibration"):
        assert opt in r.stdout, opt


def test_fp8_queries_need_fp8_keys():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--q-fp8", "--no-cpu"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--key-fp8" in r.stderr
    assert r.stdout.strip() == ""
