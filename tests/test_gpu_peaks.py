"""GPU checks of the measurement probes (libgr_peaks.so): the copy copies,
the read reduces what it reads, the exp2 chains reach the fixed point of
x = 2^-x, and the MFMA chains are deterministic and finite."""
import ctypes
import os

import numpy as np
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "shared_prefix_beam_amd", "libgr_peaks.so")
X_STAR = 0.6411857445049859          # the solution of x = 2^-x


@pytest.fixture(scope="module")
def lib():
    import torch
    torch.cuda.init()
    L = ctypes.CDLL(LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.gr_peak_mfma.argtypes = [P, I32, I32, P]
    L.gr_peak_exp2.argtypes = [P, I32, I32, P]
    L.gr_peak_copy.argtypes = [P, P, I64, I32, P]
    L.gr_peak_read.argtypes = [P, I64, P, I32, P]
    return L


def test_copy_and_read(lib):
    import torch
    log("[peaks] copy and read, 1 MiB + 48 B")
    n16 = (1 << 16) + 3                          # a ragged tail past the grid stride
    src = torch.randint(0, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    out = torch.zeros(8 * 256, dtype=torch.int32, device="cuda")
    assert lib.gr_peak_copy(src.data_ptr(), dst.data_ptr(), n16, 8, None) == 0
    assert lib.gr_peak_read(src.data_ptr(), n16, out.data_ptr(), 8, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    a = src.cpu().numpy().view(np.uint32)
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(a)


def test_exp2_reaches_fixed_point(lib):
    import torch
    log("[peaks] exp2 chains")
    out = torch.zeros(4 * 256, dtype=torch.float32, device="cuda")
    assert lib.gr_peak_exp2(out.data_ptr(), 4, 200, None) == 0
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy(), 8 * X_STAR, rtol=1e-5)


def test_mfma_deterministic(lib):
    import torch
    log("[peaks] mfma chains")
    a = torch.zeros(4 * 256, dtype=torch.float32, device="cuda")
    b = torch.zeros_like(a)
    assert lib.gr_peak_mfma(a.data_ptr(), 4, 50, None) == 0
    assert lib.gr_peak_mfma(b.data_ptr(), 4, 50, None) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and torch.equal(a, b) and float(a.abs().sum()) > 0
