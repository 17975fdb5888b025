"""bench.py's command-line contract on the CPU: it measures one GPU's share,
so a request for more GPUs is refused with a message (exit status 2) before
anything is imported or launched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*argv):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run("--gpus", n)
        assert r.returncode == 2, r
        assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout == ""
