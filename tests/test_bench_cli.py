"""The benchmark's command line on the CPU: it measures one GPU only, so a
request for more exits with a message before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps",
                        "1", "--warmup", "0"], capture_output=True, text=True, timeout=120,
                       cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)
