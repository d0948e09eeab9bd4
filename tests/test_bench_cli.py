"""bench.py's command line on the host (no GPU): more than one GPU is refused with a
message before anything touches a device, and the options parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + list(args),
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_workload_options():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--steps", "--warmup", "--graph", "--split"):
        assert opt in r.stdout
