"""Comparison of a device beam selection with the fp64 oracle, shared by the
unconstrained and the trie-constrained GPU tests.

The device ranks fp32 values and the oracle fp64 ones, so candidates whose
values lie within rounding of each other may legitimately swap.  The checks:
every device score equals the oracle's value of the same (parent, token)
within TOL; ranks whose oracle value is separated from both neighbours by
more than 2*TOL hold exactly the oracle's candidate; the device set is a
top-K within 2*TOL (nothing left out beats anything kept by more than that);
the device order is by its own score, then flat index; padding is exact.
With trie nodes, every kept beam's node equals the oracle's node of the same
candidate.
"""
import numpy as np

from gpu_util import log

# fp32 value = score + logit - LSE with |value| < 64: a few ulp (4e-6 each)
# from the additions, plus the fp32 log-sum-exp's relative error (sum of up to
# 16384 terms in a 256-thread tree, fast exp/log) amplified by nothing: the
# LSE enters additively.  1e-4 leaves a factor >10 of margin.
TOL = 1e-4
MARGIN = 64


def check_against_oracle(si, gpu, K_max, what, oracle, n_cand=None):
    """`oracle(row_offset_new)` returns the oracle's selection for those kept
    counts; `n_cand[b]` is request b's candidate count (W * V unconstrained)."""
    score, parent, token = gpu[:3]
    node = gpu[3] if len(gpu) > 3 else None
    ro, rn = si.row_offset_old, si.row_offset_new
    B, V = len(ro) - 1, si.V
    W = np.diff(ro).astype(np.int64)
    K = np.diff(rn).astype(np.int64)
    if n_cand is None:
        n_cand = W * V
    # the oracle's best K + MARGIN of every request
    wide = np.minimum(K + MARGIN, n_cand)
    rw = np.zeros(B + 1, dtype=np.int64)
    rw[1:] = np.cumsum(wide)
    ref = oracle(rw)
    o_score, o_parent, o_token = ref[:3]
    o_node = ref[3] if len(ref) > 3 else None
    for b in range(B):
        k0, k1 = int(rn[b]), int(rn[b + 1])
        n_real = int(min(K[b], K_max, n_cand[b]))
        g_s, g_p, g_t = score[k0:k1], parent[k0:k1], token[k0:k1]
        tag = f"{what} request {b} (W={W[b]}, K={K[b]})"
        # padding
        assert np.all(g_s[n_real:] == -np.inf) and np.all(g_p[n_real:] == -1) \
            and np.all(g_t[n_real:] == -1), f"{tag}: padding"
        if node is not None:
            assert np.all(node[k0:k1][n_real:] == -1), f"{tag}: node padding"
        if n_real == 0:
            continue
        g_s, g_p, g_t = g_s[:n_real], g_p[:n_real], g_t[:n_real]
        assert np.all((g_p >= 0) & (g_p < W[b]) & (g_t >= 0) & (g_t < V)), f"{tag}: range"
        g_flat = g_p.astype(np.int64) * V + g_t
        assert np.unique(g_flat).size == n_real, f"{tag}: repeated candidate"
        # device order: score descending, then flat index ascending
        assert np.all(g_s[1:] <= g_s[:-1]), f"{tag}: scores not descending"
        eq = g_s[1:] == g_s[:-1]                  # -inf == -inf counts as a tie
        assert np.all(np.diff(g_flat)[eq] > 0), f"{tag}: tie order"
        # oracle values of the device's candidates
        w0, w1 = int(rw[b]), int(rw[b + 1])
        o_flat = o_parent[w0:w1].astype(np.int64) * V + o_token[w0:w1]
        o_val = o_score[w0:w1]
        pos = {int(f): i for i, f in enumerate(o_flat)}
        missing = [int(f) for f in g_flat if int(f) not in pos]
        assert not missing, f"{tag}: {len(missing)} device picks outside the oracle's best " \
                            f"{w1 - w0}"
        idx = np.array([pos[int(f)] for f in g_flat])
        u = o_val[idx]
        if node is not None:
            assert np.array_equal(node[k0:k0 + n_real], o_node[w0:w1][idx]), f"{tag}: nodes"
        fin = np.isfinite(u)
        assert np.array_equal(np.isfinite(g_s), fin), f"{tag}: -inf mismatch"
        err = np.abs(g_s[fin].astype(np.float64) - u[fin])
        assert err.size == 0 or err.max() <= TOL, f"{tag}: score error {err.max():.3g}"
        # a top-K within 2*TOL: what the oracle keeps and the device drops
        # is no better than the device's worst pick by more than that
        dropped = np.setdiff1d(np.arange(n_real), idx)
        if dropped.size:
            assert o_val[dropped].max() <= u.min() + 2 * TOL, f"{tag}: set"
        # separated ranks are unique: exact match there
        ext = np.concatenate([[np.inf], o_val, [-np.inf]])
        with np.errstate(invalid="ignore"):       # inf - inf: not separated
            gap_hi = ext[:-2][:n_real] - o_val[:n_real]
            gap_lo = o_val[:n_real] - ext[2:][:n_real]
        sep = (gap_hi > 2 * TOL) & (gap_lo > 2 * TOL)
        assert np.array_equal(g_flat[sep], o_flat[:n_real][sep]), f"{tag}: rank mismatch"
        log(f"  {tag}: {int(sep.sum())}/{n_real} ranks separated and equal, "
            f"max err {0 if err.size == 0 else err.max():.2e}")


