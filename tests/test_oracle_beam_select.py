"""Pins of the beam-selection oracle (log_softmax + top-K over beams x
vocabulary) and planted mistakes in copies of it (CPU only)."""
import inspect
import math
import textwrap

import numpy as np
import pytest

from oracle import oracle as O


def brute(row_offset_old, row_offset_new, score_old, logits):
    """Enumeration with Python floats: log-softmax from math.exp / math.log
    per row, candidates ordered by sorted() on (-value, flat index)."""
    B = len(row_offset_new) - 1
    V = len(logits[0]) if len(logits) else 0
    out = []
    for b in range(B):
        r0, r1 = row_offset_old[b], row_offset_old[b + 1]
        cands = []
        for w in range(r1 - r0):
            row = [float(x) for x in logits[r0 + w]]
            m = max(row)
            lse = m + math.log(sum(math.exp(x - m) for x in row))
            for v, x in enumerate(row):
                cands.append((-(float(score_old[r0 + w]) + x - lse), w * V + v))
        cands.sort()
        k = row_offset_new[b + 1] - row_offset_new[b]
        for i in range(k):
            if i < len(cands):
                out.append((-cands[i][0], cands[i][1] // V, cands[i][1] % V))
            else:
                out.append((-math.inf, -1, -1))
    return out


def check_against_brute(fn, ro, rn, s, x):
    got = fn(ro, rn, s, x)
    ref = brute(list(ro), list(rn), s, x)
    assert len(got[0]) == len(ref)
    for i, (val, p, t) in enumerate(ref):
        assert got[1][i] == p and got[2][i] == t, (i, got[1][i], got[2][i], p, t)
        if math.isinf(val):
            assert got[0][i] == val
        else:
            assert abs(got[0][i] - val) < 1e-12


def pin_bruteforce(fn, seed=0):
    rng = np.random.default_rng(seed)
    for trial in range(6):
        B = int(rng.integers(1, 4))
        W_old = rng.integers(0, 5, size=B)
        W_new = rng.integers(0, 9, size=B)
        ro = np.concatenate([[0], np.cumsum(W_old)]).astype(np.int32)
        rn = np.concatenate([[0], np.cumsum(W_new)]).astype(np.int32)
        V = int(rng.integers(1, 7))
        s = rng.standard_normal(int(ro[-1])) * 2
        x = rng.standard_normal((int(ro[-1]), V)) * 3
        check_against_brute(fn, ro, rn, s, x)


def pin_closed_forms(fn):
    # equal logits: every candidate of a row is score - ln V; all kept in index order
    V = 5
    ro = np.array([0, 2]); rn = np.array([0, 10])
    s = np.array([-1.0, -1.0]); x = np.full((2, V), 0.7)
    val, p, t = fn(ro, rn, s, x)
    assert np.allclose(val, -1.0 - math.log(V), atol=1e-14)
    assert list(p) == [0] * 5 + [1] * 5 and list(t) == list(range(5)) * 2
    # more slots than candidates: tail is (-inf, -1, -1)
    val, p, t = fn(np.array([0, 1]), np.array([0, 4]), np.array([0.0]), np.array([[0.0, 1.0]]))
    assert list(p) == [0, 0, -1, -1] and list(t) == [1, 0, -1, -1] and np.isinf(val[2:]).all()


def pin_shift_invariance(fn, seed=1):
    rng = np.random.default_rng(seed)
    ro = np.array([0, 6]); rn = np.array([0, 9])
    s = rng.standard_normal(6); x = rng.standard_normal((6, 11))
    a = fn(ro, rn, s, x)
    b = fn(ro, rn, s, x + rng.standard_normal((6, 1)) * 5)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    assert np.allclose(a[0], b[0], atol=1e-12)


def battery(fn):
    failed = []
    for name, pin in (("brute", pin_bruteforce), ("closed", pin_closed_forms),
                      ("shift", pin_shift_invariance)):
        try:
            pin(fn)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            failed.append(name)
    return failed


def test_bruteforce():
    pin_bruteforce(O.beam_select)


def test_closed_forms():
    pin_closed_forms(O.beam_select)


def test_shift_invariance():
    pin_shift_invariance(O.beam_select)


MUTANTS = [
    ("log-softmax normaliser dropped", "value = (score_old[r0:r1, None] + x - lse).ravel()",
     "value = (score_old[r0:r1, None] + x).ravel()"),
    ("max only, no log-sum", "lse = m + np.log(np.exp(x - m).sum(axis=1, keepdims=True))",
     "lse = m"),
    ("ties broken by larger index", "order = np.lexsort((flat, -value))",
     "order = np.lexsort((-flat, -value))"),
    ("ascending selection", "order = np.lexsort((flat, -value))",
     "order = np.lexsort((flat, value))"),
    ("parent and token swapped", "parent[k0:k0 + n] = sel // V",
     "parent[k0:k0 + n] = sel % V"),
    ("score of the first beam for all", "value = (score_old[r0:r1, None] + x - lse).ravel()",
     "value = (score_old[r0] + x - lse).ravel()"),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(name, orig, bad):
    src = textwrap.dedent(inspect.getsource(O.beam_select))
    assert orig in src
    ns = {"np": np, "math": math}
    exec(src.replace(orig, bad, 1), ns)
    assert battery(ns["beam_select"]), f"no pin rejects '{name}'"


def test_real_oracle_passes_battery():
    assert battery(O.beam_select) == []
