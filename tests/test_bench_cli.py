"""bench.py's command line without a GPU: more than one GPU is refused with a
message and a nonzero status, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_legs():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--no-warm", "--profile-run", "--profile-groups", "--no-cpu-baseline",
                 "--no-probe"):
        assert flag in r.stdout
