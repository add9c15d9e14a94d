"""GPU parity on seeded random shapes.

Each case draws the request count, the beams of each request (some requests
empty), context and BeamKV lengths, the group size, the head dim, duplicate
beam paths and the query scale, then compares every row of the library's
planned path with the fp64 oracle.  Every other case also runs through a
paged context of a random page size (a multiple of 16), against the oracle and
bitwise against the dense call.  The planner picks 16-row or 32-row waves and
context splits by itself, so the draws reach decompositions that the
hand-written cases do not name.
"""
import numpy as np
import pytest

from gpu_util import assert_parity, log, run_lib
from oracle import oracle as O
from shared_prefix_beam_amd import inputs as I
from test_gpu_paged import run_paged

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw(seed):
    """(D, Hq, Hkv, B, W, ctx_len, beam_len, kwargs) of case `seed`."""
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Hkv = max(1, min(Hkv, 32 // G))               # at most 32 query heads
    B = int(rng.integers(1, 5))
    W = [int(x) for x in rng.integers(0, 161, size=B)]
    if max(W) == 0:
        W[0] = 1
    ctx_len = [int(x) for x in rng.integers(0, 3001, size=B)]
    beam_len = [int(x) for x in rng.integers(0, 7, size=B)]
    kw = dict(dup_frac=float(rng.choice([0.0, 0.3])), q_std=float(rng.choice([1.0, 4.0])))
    return D, G * Hkv, Hkv, B, W, ctx_len, beam_len, kw


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    D, Hq, Hkv, B, W, L, T, kw = draw(seed)
    inp = I.custom(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, ctx_len=L, beam_len=T, seed=seed, **kw)
    log(f"[random {seed}] D={D} Hq={Hq} Hkv={Hkv} W={W} L={L} T={T} {kw}")
    out, lse = run_lib(inp, "fused")
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"random {seed}")
    if seed % 2 == 0:
        page = 16 * int(np.random.default_rng(seed).integers(1, 9))
        pg = I.to_paged(inp, page, seed=seed + 1)
        log(f"[random {seed}] paged, page size {page}")
        p_out, p_lse = run_paged(inp, pg)
        assert_parity(p_out, p_lse, ref_out, ref_lse, f"random {seed} paged")
        assert np.array_equal(p_out, out) and np.array_equal(p_lse, lse), \
            "paged and dense results differ"
