"""bench.py's command line on the CPU: more than one GPU is refused with a
message and exit status 2, before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout == ""
