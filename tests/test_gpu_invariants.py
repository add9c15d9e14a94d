"""GPU invariants that need no oracle: determinism, permutation
equivariance, duplicate rows, NaN padding, the metadata checker."""
import numpy as np
import pytest

from gpu_util import log, run_lib
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_run_to_run_bitwise_determinism():
    inp = I.generate(I.WORKLOADS[2])
    log("[invariant] determinism on workload 2")
    dev = I.to_torch(inp)
    a = run_lib(inp, dev=dev)
    b = run_lib(inp, dev=dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_row_permutation_is_equivariant():
    """Permuting a request's beams (q rows and path rows together) permutes
    the outputs bitwise: every query column is computed by the same sequence
    of operations whatever its position in the stack."""
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[50, 33], ctx_len=[300, 128], beam_len=[3, 2],
                   seed=3)
    log("[invariant] permutation")
    out, lse = run_lib(inp)
    rng = np.random.default_rng(0)
    perm = np.arange(inp.R)
    for b in range(inp.B):
        r0, r1 = int(inp.row_offset[b]), int(inp.row_offset[b + 1])
        perm[r0:r1] = r0 + rng.permutation(r1 - r0)
    inp.q[:] = inp.q[perm]
    inp.beam_path[:] = inp.beam_path[perm]
    out2, lse2 = run_lib(inp)
    assert np.array_equal(out2, out[perm]) and np.array_equal(lse2, lse[perm])


def test_identical_rows_give_identical_outputs():
    inp = I.custom(B=1, Hq=16, Hkv=8, D=128, W=[64], ctx_len=[500], beam_len=[3], seed=5,
                   dup_frac=0.3)
    src = inp.dup_src[0]
    for w in inp.dup_rows[0]:
        inp.q[w] = inp.q[src]
    log("[invariant] duplicate (q, path) rows")
    out, lse = run_lib(inp)
    for w in inp.dup_rows[0]:
        assert np.array_equal(out[w], out[src]) and np.array_equal(lse[w], lse[src])


def test_outputs_finite_with_nan_padding():
    for cfg in (3, 5):
        inp = I.generate(I.WORKLOADS[cfg])
        log(f"[invariant] NaN padding, workload {cfg}")
        out, lse = run_lib(inp)
        assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_fused_matches_generic_comparator():
    inp = I.generate(I.WORKLOADS[4])
    log("[invariant] fused vs generic on workload 4")
    dev = I.to_torch(inp)
    a = run_lib(inp, "fused", dev=dev)
    b = run_lib(inp, "generic", dev=dev)
    assert np.max(np.abs(a[0] - b[0])) <= 2e-2
    assert np.max(np.abs(a[1] - b[1])) <= 1e-3


def test_metadata_checker():
    import torch
    from shared_prefix_beam_amd import gr_attn
    inp = I.generate(I.WORKLOADS[5])
    dev = I.to_torch(inp)
    kw = dict(B=inp.B, R=inp.R, Hq=inp.wl.Hq, Hkv=inp.wl.Hkv, D=inp.wl.D, W_max=max(inp.wl.W),
              ctx_cap=inp.ctx_cap, beam_cap=inp.beam_cap)
    log("[invariant] metadata checker")
    v = gr_attn.check_metadata(dev["ctx_len"], dev["beam_path"], dev["beam_len"],
                               dev["row_offset"], **kw)
    torch.cuda.synchronize()
    assert int(v.item()) == 0
    bad_path = dev["beam_path"].clone()
    bad_path[3, 0] = inp.beam_cap          # one past the end
    bad_path[10, 1] = -1
    bad_len = dev["ctx_len"].clone()
    bad_len[2] = inp.ctx_cap + 1
    v = gr_attn.check_metadata(bad_len, bad_path, dev["beam_len"], dev["row_offset"], **kw)
    torch.cuda.synchronize()
    assert int(v.item()) == 3
