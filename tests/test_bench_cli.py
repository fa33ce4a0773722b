"""bench.py's command line, host only: it measures one GPU, so --gpus N with N > 1
exits with status 2 and says why, before touching torch or the device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                           text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2, (n, r.returncode, r.stderr[-500:])
        assert "measures one GPU" in r.stderr and r.stdout == ""
