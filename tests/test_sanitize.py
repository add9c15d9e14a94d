"""The host-side C code under AddressSanitizer and UndefinedBehaviorSanitizer
on the CPU: the C ABI's validation, work decomposition and workspace layout
(launchers stubbed to check each planned launch against the caller's
buffers), and the C oracle on small random inputs (tests/sanitize/)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_sanitizers(tmp_path):
    res = subprocess.run(["bash", os.path.join(HERE, "sanitize", "build_and_run.sh"),
                          str(tmp_path)], capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "SANITIZE_OK" in res.stdout, tail
    assert "runtime error" not in res.stderr, tail
