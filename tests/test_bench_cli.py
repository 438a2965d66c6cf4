"""bench.py's command line on the CPU: it measures one GPU only and says so for
--gpus above 1, and refuses a step count below one.  Both exits happen before
anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_zero_steps_are_refused():
    r = _bench("--steps", "0")
    assert r.returncode == 2
    assert "--steps must be at least 1" in r.stderr
