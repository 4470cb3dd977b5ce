"""Host-side contract of bench.py, no GPU needed: one GPU only (a larger --gpus is refused with
a message and exit status 2, before anything touches a device), and the documented flags."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run("--gpus", n)
        assert r.returncode == 2
        assert f"--gpus {n}" in r.stderr and "not supported" in r.stderr
        assert r.stdout == ""


def test_flags():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--skip-cpu-baseline", "--skip-decode", "--decode-only",
                 "--traffic-copy-mib"):
        assert flag in r.stdout
