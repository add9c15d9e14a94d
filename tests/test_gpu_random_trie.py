"""GPU parity of item-constrained beam selection on seeded random catalogs.

Each case draws a catalog (item count, depth, vocabulary), the decode step
(the root, a middle level or the leaves, where no token is legal), ragged
requests (some empty), a share of dead beams and the spread of logits and
scores; the result, kept beams' trie nodes included, is compared with the
fp64 oracle, which walks every beam's prefix from the root.
"""
import numpy as np
import pytest

from gpu_util import log
from test_gpu_beam_select_trie import check
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu

N_CASES = 12


def draw(seed):
    rng = np.random.default_rng(9000 + seed)
    V = int(rng.integers(50, 4001))
    depth = int(rng.integers(2, 5))
    n_items = int(rng.integers(100, 20001))
    step = int(rng.integers(0, depth + 1))
    B = int(rng.integers(1, 6))
    W_old = [int(x) for x in rng.integers(0, 201, size=B)]
    if max(W_old) == 0:
        W_old[0] = 1
    W_new = [int(x) for x in rng.integers(0, 401, size=B)]
    if max(W_new) == 0:
        W_new[0] = 1
    dead = float(rng.choice([0.0, 0.2]))
    return V, depth, n_items, step, W_old, W_new, dead


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_trie_selection(seed):
    V, depth, n_items, step, W_old, W_new, dead = draw(seed)
    trie = I.build_trie(I.sid_catalog(n_items, depth, V, seed=seed), V)
    ti = I.trie_select_inputs(W_old, W_new, V, step, trie, seed=seed + 1, dead=dead)
    log(f"[trie random {seed}] V={V} depth={depth} items={n_items} step={step} "
        f"W_old={W_old} W_new={W_new} dead={dead}")
    check(ti, max(W_new), f"random {seed}")
