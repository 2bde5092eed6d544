"""bench.py as a command: it parses, and it refuses more than one GPU with a message."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_help_lists_options():
    r = _run("--help")
    assert r.returncode == 0, r.stderr
    for opt in ("--gpus", "--steps", "--warmup", "--config", "--cpu-rows", "--no-cpu-baseline", "--traffic-probe"):
        assert opt in r.stdout


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
