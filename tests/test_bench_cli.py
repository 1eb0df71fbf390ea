"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with exit status 2 and a message, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_multi_gpu_refused():
    for n in ("2", "8"):
        r = run_bench("--gpus", n, "--steps", "1", "--warmup", "0")
        assert r.returncode == 2, (r.returncode, r.stderr)
        assert "one GPU" in r.stderr
        assert r.stdout == ""  # no JSON line


def test_help_lists_modes():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--compare-blas", "--profile-traffic",
                 "--profile-decode", "--profile-layouts", "--only"):
        assert flag in r.stdout
