"""The probe library (libgr_peaks.so) on the CPU: it loads, exports every
function gr_peaks.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gr_peaks.h")
LIB = os.path.join(ROOT, "shared_prefix_beam_amd", "libgr_peaks.so")
HIP_INVALID_VALUE = 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built")
    L = ctypes.CDLL(LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.gr_peak_mfma.argtypes = [P, I32, I32, P]
    L.gr_peak_exp2.argtypes = [P, I32, I32, P]
    L.gr_peak_copy.argtypes = [P, P, I64, I32, P]
    L.gr_peak_read.argtypes = [P, I64, P, I32, P]
    return L


def test_exports_every_declared_function(lib):
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(gr_[a-z0-9_]+)\s*\(", src)))
    assert names == ["gr_peak_copy", "gr_peak_exp2", "gr_peak_mfma", "gr_peak_read"]
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("args", [(None, 8, 10), (16, 0, 10), (16, 8, 0), (16, -1, 10)])
def test_mfma_and_exp2_reject_bad_arguments(lib, args):
    out, grid, iters = args
    assert lib.gr_peak_mfma(out, grid, iters, None) == HIP_INVALID_VALUE
    assert lib.gr_peak_exp2(out, grid, iters, None) == HIP_INVALID_VALUE


def test_copy_and_read_reject_bad_arguments(lib):
    p = 4096                                     # never dereferenced: rejected first
    assert lib.gr_peak_copy(None, p, 16, 8, None) == HIP_INVALID_VALUE
    assert lib.gr_peak_copy(p, None, 16, 8, None) == HIP_INVALID_VALUE
    assert lib.gr_peak_copy(p, p, 0, 8, None) == HIP_INVALID_VALUE
    assert lib.gr_peak_copy(p, p, 16, 0, None) == HIP_INVALID_VALUE
    assert lib.gr_peak_read(None, 16, p, 8, None) == HIP_INVALID_VALUE
    assert lib.gr_peak_read(p, 16, None, 8, None) == HIP_INVALID_VALUE
    assert lib.gr_peak_read(p, -5, p, 8, None) == HIP_INVALID_VALUE
