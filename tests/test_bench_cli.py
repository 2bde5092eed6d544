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
    for opt in ("--gpus", "--steps", "--warmup", "--config", "--cpu-rows", "--no-cpu-baseline", "--traffic-probe",
                "--headline-only", "--no-per-config", "--no-parity", "--no-memory-sweep"):
        assert opt in r.stdout


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_measured_traffic_follows_the_kernel_source():
    """`roofline.traffic` comes from the committed counter summary only while the
    engine source still hashes to what the summary records."""
    sys.path.insert(0, ROOT)
    import hashlib
    import bench
    kv = {}
    for line in open(bench.TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    digest = hashlib.sha256(open(bench.KERNEL_SRC["engine"], "rb").read()).hexdigest()
    got = bench.measured_traffic("dw_gemm")
    if kv.get("engine_sha256") == digest:
        assert got == float(kv["dw_traffic_bytes_per_launch"])
    else:
        assert got is None
    assert bench.measured_traffic("no_such_kernel") is None
