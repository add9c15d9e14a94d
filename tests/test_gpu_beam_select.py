"""GPU parity of beam selection (log_softmax + top-K over beams x vocabulary)
through the C ABI against the fp64 oracle (comparison rules in
select_check.py: exact where ranks are separated, a valid top-K within the
fp32 tolerance elsewhere, exact padding)."""
import numpy as np
import pytest

from gpu_util import log
from oracle import oracle as O
from select_check import check_against_oracle as _check
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu

def check_against_oracle(si, gpu, K_max, what):
    _check(si, gpu, K_max, what,
           lambda rw: O.beam_select(si.row_offset_old, rw, si.score_old, si.logits))


def run_gpu(si, K_max):
    import torch
    from shared_prefix_beam_amd import gr_attn
    dev = "cuda"
    R_new = int(si.row_offset_new[-1])
    out = gr_attn.beam_select(torch.from_numpy(si.row_offset_old).to(dev),
                              torch.from_numpy(si.row_offset_new).to(dev),
                              torch.from_numpy(si.score_old).to(dev),
                              torch.from_numpy(np.ascontiguousarray(si.logits)).to(dev),
                              K_max, R_new=R_new)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in out)


def select_case(W_old, W_new, V, seed, K_max=None, **kw):
    si = I.select_inputs(W_old, W_new, V, seed, **kw)
    K_max = K_max if K_max is not None else max(max(W_new), 1)
    return si, K_max


def test_ragged_small():
    """Ragged requests: no old beams, no kept beams, fewer rows than K (no
    bound), one row, V not a multiple of the 256-thread tile."""
    si, K_max = select_case([3, 0, 7, 1, 5, 2], [4, 2, 0, 9, 5, 40], V=300, seed=1)
    log("[select] ragged small")
    check_against_oracle(si, run_gpu(si, K_max), K_max, "ragged")


def test_fewer_candidates_than_kept():
    """W*V < K: every candidate is kept, then (-inf, -1, -1) padding."""
    si, K_max = select_case([1, 2], [9, 7], V=3, seed=2)
    log("[select] fewer candidates than kept")
    check_against_oracle(si, run_gpu(si, K_max), K_max, "short")


def test_vocabulary_of_one():
    si, K_max = select_case([4, 3], [2, 3], V=1, seed=3)
    log("[select] V=1")
    check_against_oracle(si, run_gpu(si, K_max), K_max, "V=1")


def test_kept_beyond_k_max_is_padded():
    """A request keeping more than K_max beams gets the best K_max, then
    padding (the documented clamp)."""
    si = I.select_inputs([5, 6], [3, 9], V=50, seed=4)
    log("[select] K > K_max clamp")
    check_against_oracle(si, run_gpu(si, 6), 6, "clamp")


def test_exact_ties_break_by_index():
    """Logits on a coarse grid: many exact ties inside a row, ranked by token
    index on both sides."""
    si = I.select_inputs([6, 9], [40, 25], V=700, seed=5)
    si.logits = np.round(si.logits * 2) / 2
    si.score_old[:] = np.float32(-1.0)
    log("[select] exact ties")
    check_against_oracle(si, run_gpu(si, 40), 40, "ties")


def test_masked_vocabulary():
    """Most logits -inf (a constrained vocabulary): finite candidates first,
    then -inf ones by flat index once the finite ones run out."""
    si = I.select_inputs([4, 3], [30, 200], V=500, seed=6)
    rng = np.random.default_rng(7)
    mask = rng.random(si.logits.shape) < 0.9
    mask[:, 0] = False                            # every row keeps a finite logit
    si.logits[mask] = -np.inf
    log("[select] masked vocabulary")
    check_against_oracle(si, run_gpu(si, 200), 200, "masked")


def test_many_rows_few_kept():
    """W much larger than K: the bound comes from the rows' heads."""
    si, K_max = select_case([2000, 700], [4, 1], V=1000, seed=8)
    log("[select] many rows, few kept")
    check_against_oracle(si, run_gpu(si, K_max), K_max, "wide")


def test_maximum_sizes():
    """V = 16384 and K = K_max = 1024, beside a small request."""
    si = I.select_inputs([1100, 3], [1024, 17], V=16384, seed=9)
    log("[select] V=16384, K=1024")
    check_against_oracle(si, run_gpu(si, 1024), 1024, "max")


@pytest.mark.parametrize("cfg", sorted(I.SELECT_WORKLOADS))
def test_select_workloads(cfg):
    """The benchmarked shapes (W=128 x 8 requests, W=900 x 4, V=8192)."""
    si = I.select_workload(cfg)
    log(f"[select] workload {I.SELECT_WORKLOADS[cfg]['name']}")
    K_max = int(np.diff(si.row_offset_new).max())
    check_against_oracle(si, run_gpu(si, K_max), K_max, I.SELECT_WORKLOADS[cfg]["name"])


def test_repeatable():
    """Two calls on the same inputs give bitwise-equal outputs."""
    si, K_max = select_case([128] * 3, [128] * 3, V=4096, seed=10)
    a, b = run_gpu(si, K_max), run_gpu(si, K_max)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.int32), y.view(np.int32))


def test_dominant_rows_are_selected_again():
    """Two rows far above the rest: their whole 32-key lists clear the bound,
    so they are selected again from their logits, and every kept beam comes
    from them."""
    si = I.select_inputs([50, 9], [200, 3], V=1000, seed=11)
    si.score_old[:50] = np.float32(-60.0)
    si.score_old[[7, 31]] = np.float32(0.0)
    log("[select] dominant rows")
    gpu = run_gpu(si, 200)
    check_against_oracle(si, gpu, 200, "dominant")
    assert set(np.unique(gpu[1][:200]).tolist()) == {7, 31}


def test_no_bound_many_survivors():
    """Fewer head keys than kept beams (no bound): every row is selected
    again and the survivors (127 x 1024) exceed what the workgroup keeps in
    LDS and registers."""
    si = I.select_inputs([127], [1024], V=2000, seed=12)
    log("[select] no bound, many survivors")
    check_against_oracle(si, run_gpu(si, 1024), 1024, "nobound")
