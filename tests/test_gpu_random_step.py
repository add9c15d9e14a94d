"""GPU parity of the beam step on seeded random shapes: bit-exact against the
oracle, the out-of-range count included.

Each case draws the request count, KV heads, head dim, the beams before and
after the step (either may be zero), the path lengths and the capacities;
T_cap is sometimes the longest path itself, so the step of that request is out
of range and both sides must count it and leave its state alone.
"""
import numpy as np
import pytest

from gpu_util import log
from oracle import oracle as O
from test_gpu_beam_step import assert_same, gpu_step
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu

N_CASES = 12


def draw(seed):
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 7))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    W_old = [int(x) for x in rng.integers(0, 301, size=B)]
    W_new = [int(x) for x in rng.integers(0, 301, size=B)]
    beam_len = [int(x) for x in rng.integers(0, 7, size=B)]
    T_cap = max(beam_len) + int(rng.integers(0, 3))
    T_cap = max(T_cap, 1)
    W_cap = max(max(W_old), max(W_new), 1) + int(rng.integers(0, 5))
    return B, Hkv, D, W_old, W_new, beam_len, T_cap, W_cap


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_step(seed):
    B, Hkv, D, W_old, W_new, beam_len, T_cap, W_cap = draw(seed)
    st = I.step_inputs(B=B, Hkv=Hkv, D=D, W_old=W_old, W_new=W_new, beam_len=beam_len, seed=seed,
                       T_cap=T_cap, W_cap=W_cap)
    log(f"[step random {seed}] Hkv={Hkv} D={D} W_old={W_old} W_new={W_new} T={beam_len} "
        f"T_cap={T_cap} W_cap={W_cap}")
    s = st.state
    path_init = np.full((st.R_new, s.T_cap), -1, dtype=np.int32)
    args = (s.row_offset, st.row_offset_new, st.parent, s.beam_path, s.beam_len, st.new_k,
            st.new_v, path_init, s.beam_k, s.beam_v, s.W_cap)
    assert_same(gpu_step(*args), O.beam_step(*args), f"random step {seed}")


def test_many_small_requests_step():
    """120 requests of 0-8 beams before and after the step, bit-exact."""
    rng = np.random.default_rng(120)
    B = 120
    W_old = [int(x) for x in rng.integers(0, 9, size=B)]
    W_new = [int(x) for x in rng.integers(0, 9, size=B)]
    beam_len = [int(x) for x in rng.integers(0, 5, size=B)]
    st = I.step_inputs(B=B, Hkv=8, D=128, W_old=W_old, W_new=W_new, beam_len=beam_len, seed=121,
                       T_cap=5, W_cap=9)
    log("[step] 120 small requests")
    s = st.state
    path_init = np.full((st.R_new, s.T_cap), -1, dtype=np.int32)
    args = (s.row_offset, st.row_offset_new, st.parent, s.beam_path, s.beam_len, st.new_k,
            st.new_v, path_init, s.beam_k, s.beam_v, s.W_cap)
    assert_same(gpu_step(*args), O.beam_step(*args), "120 small requests")
