"""GPU parity of beam selection on seeded random shapes.

Each case draws the request count, the beams before the step and the beams
kept per request (either may be zero), the vocabulary size (from one token up
to the largest supported, so both the one-wave and the workgroup row kernels
run), K_max (sometimes below a request's kept count, which pads), and the
spread of logits and scores; the result is compared with the fp64 oracle under
the rules of select_check.py.
"""
import numpy as np
import pytest

from gpu_util import log
from test_gpu_beam_select import check_against_oracle, run_gpu
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu

N_CASES = 16


def draw(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 7))
    V = int(np.exp(rng.uniform(0.0, np.log(16384))))
    V = max(1, min(V, 16384))
    W_old = [int(x) for x in rng.integers(0, 401, size=B)]
    W_new = [int(min(x, 1024)) for x in rng.integers(0, 1025, size=B)]
    if max(W_new) == 0:
        W_new[0] = 1
    K_max = max(W_new) if rng.random() < 0.7 else max(1, int(rng.integers(1, max(W_new) + 1)))
    kw = dict(logit_std=float(rng.choice([0.5, 2.0, 8.0])),
              score_spread=float(rng.choice([0.1, 3.0, 20.0])))
    return W_old, W_new, V, K_max, kw


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_selection(seed):
    W_old, W_new, V, K_max, kw = draw(seed)
    si = I.select_inputs(W_old, W_new, V, seed, **kw)
    log(f"[select random {seed}] W_old={W_old} W_new={W_new} V={V} K_max={K_max} {kw}")
    check_against_oracle(si, run_gpu(si, K_max), K_max, f"random {seed}")


def test_many_small_requests():
    """150 requests of 0-8 beams before and 0-12 kept (one request-stage
    workgroup each), against the oracle."""
    rng = np.random.default_rng(150)
    W_old = [int(x) for x in rng.integers(0, 9, size=150)]
    W_new = [int(x) for x in rng.integers(0, 13, size=150)]
    si = I.select_inputs(W_old, W_new, 700, 150)
    K_max = max(W_new)
    log(f"[select] 150 small requests, V=700, K_max={K_max}")
    check_against_oracle(si, run_gpu(si, K_max), K_max, "150 small requests")
