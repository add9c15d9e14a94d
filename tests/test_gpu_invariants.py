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


def count_violations(row_offset, ctx_len, beam_len, beam_path, *, B, R, W_max, ctx_cap, T_cap,
                     beam_cap):
    """The documented preconditions of gr_check_metadata, counted per request
    (row range, context length, path length; plus one for a first offset
    other than 0 or a last other than R) and per used path entry."""
    bad = 0
    for b in range(B):
        lo, hi = int(row_offset[b]), int(row_offset[b + 1])
        bad += int(hi < lo or hi - lo > W_max or lo < 0 or hi > R)
        bad += int(not 0 <= ctx_len[b] <= ctx_cap)
        bad += int(not 0 <= beam_len[b] <= T_cap)
    if B > 0:
        bad += int(row_offset[0] != 0 or row_offset[B] != R)
    for t in range(R if B > 0 else 0):
        b = 0
        while b + 1 < B and row_offset[b + 1] <= t:   # the row's request, as found
            b += 1
        T = min(max(int(beam_len[b]), 0), T_cap)
        bad += int(np.sum((beam_path[t, :T] < 0) | (beam_path[t, :T] >= beam_cap)))
    return bad


@pytest.mark.parametrize("seed", range(8))
def test_metadata_checker_counts_every_rule(seed):
    """Seeded corruptions of the row offsets, lengths and path entries: the
    device count equals the count of the documented rules."""
    import torch
    from shared_prefix_beam_amd import gr_attn
    inp = I.generate(I.WORKLOADS[3])
    rng = np.random.default_rng(600 + seed)
    ro, cl, bl = inp.row_offset.copy(), inp.ctx_len.copy(), inp.beam_len.copy()
    bp = inp.beam_path.copy()
    B, R, T_cap = inp.B, inp.R, bp.shape[1]
    W_max = int(np.diff(inp.row_offset).max())
    for _ in range(int(rng.integers(1, 4))):
        kind = int(rng.integers(0, 6))
        b = int(rng.integers(0, B))
        if kind == 0:
            ro[b + 1] = ro[b] - int(rng.integers(1, 5))          # decreasing
        elif kind == 1:
            ro[int(rng.integers(0, B + 1))] += int(rng.integers(1, 40))   # too wide / past R
        elif kind == 2:
            cl[b] = -1 if rng.random() < 0.5 else inp.ctx_cap + 1
        elif kind == 3:
            bl[b] = -1 if rng.random() < 0.5 else T_cap + 1
        elif kind == 4:
            bp[int(rng.integers(0, R)), 0] = -1
        else:
            bp[int(rng.integers(0, R)), int(rng.integers(0, T_cap))] = inp.beam_cap
    kw = dict(B=B, R=R, W_max=W_max, ctx_cap=inp.ctx_cap, T_cap=T_cap, beam_cap=inp.beam_cap)
    want = count_violations(ro, cl, bl, bp, **kw)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    log(f"[invariant] metadata checker, corruption seed {seed}: {want} violations expected")
    ckw = {k: x for k, x in kw.items() if k != "T_cap"}   # T_cap: the path table's stride
    v = gr_attn.check_metadata(dev(cl), dev(bp), dev(bl), dev(ro), Hq=inp.wl.Hq, Hkv=inp.wl.Hkv,
                               D=inp.wl.D, **ckw)
    torch.cuda.synchronize()
    assert int(v.item()) == want
    assert want > 0 or seed < 0
