"""Pins of the trie-constrained selection oracle (prefix traversal of a CSR
semantic-ID trie, legal-token log-softmax, top-K over beams) and planted
mistakes in copies of it (CPU only)."""
import inspect
import math
import textwrap

import numpy as np
import pytest

from oracle import oracle as O
from shared_prefix_beam_amd import inputs as I


def legal_from_items(items, prefix):
    """Legal next tokens of a prefix read straight off the item list: the
    token after the prefix in every item that starts with it (no trie)."""
    s = len(prefix)
    out = set()
    for it in items:
        if s < len(it) and all(int(it[j]) == int(prefix[j]) for j in range(s)):
            out.add(int(it[s]))
    return sorted(out)


def brute(items, ro, rn, score_old, logits, sid):
    """Enumeration with Python floats over the item list: a beam's legal
    tokens, their log-softmax over that set (math.exp / math.log), candidates
    ordered by sorted() on (-value, flat index)."""
    V = len(logits[0])
    out = []
    for b in range(len(rn) - 1):
        r0, r1 = ro[b], ro[b + 1]
        cands = []
        for w in range(r1 - r0):
            legal = legal_from_items(items, sid[r0 + w])
            if not legal:
                continue
            xs = [float(logits[r0 + w][t]) for t in legal]
            m = max(xs)
            lse = m + math.log(sum(math.exp(x - m) for x in xs))
            for t, x in zip(legal, xs):
                cands.append((-(float(score_old[r0 + w]) + x - lse), w * V + t))
        cands.sort()
        for i in range(rn[b + 1] - rn[b]):
            if i < len(cands):
                out.append((-cands[i][0], cands[i][1] // V, cands[i][1] % V))
            else:
                out.append((-math.inf, -1, -1))
    return out


def tiny_case(rng, V=6, depth=3, n_items=20, B=3, step=None):
    items = I.sid_catalog(n_items, depth, V, int(rng.integers(1 << 30)))
    trie = I.build_trie(items, V)
    W_old = rng.integers(0, 5, size=B)
    W_new = rng.integers(0, 12, size=B)
    ro = np.concatenate([[0], np.cumsum(W_old)]).astype(np.int32)
    rn = np.concatenate([[0], np.cumsum(W_new)]).astype(np.int32)
    R = int(ro[-1])
    s = step if step is not None else int(rng.integers(0, depth + 1))
    sid = items[rng.integers(0, items.shape[0], size=R), :s].reshape(R, s)
    if R and s:                                   # some prefixes leave the trie
        junk = rng.random(R) < 0.25
        sid[junk] = rng.integers(0, V, size=(int(junk.sum()), s))
    score = rng.standard_normal(R) * 2
    x = rng.standard_normal((R, V)) * 3
    return items, trie, ro, rn, score, x, sid


def call(fn, trie, ro, rn, s, x, sid):
    return fn(ro, rn, s, x, sid, trie.node_ptr, trie.edge_tok, trie.edge_child)


def pin_bruteforce(fn, seed=0):
    """Against enumeration over the raw item list; the kept beam's node is
    checked with the catalog's own prefix lookup (no trie walk)."""
    rng = np.random.default_rng(seed)
    for trial in range(8):
        items, trie, ro, rn, s, x, sid = tiny_case(rng)
        got = call(fn, trie, ro, rn, s, x, sid)
        ref = brute(items, list(ro), list(rn), s, x, sid)
        assert len(got[0]) == len(ref)
        for i, (val, p, t) in enumerate(ref):
            assert got[1][i] == p and got[2][i] == t, (trial, i)
            if math.isinf(val):
                assert got[0][i] == val and got[3][i] == -1
            else:
                assert abs(got[0][i] - val) < 1e-12
                b = int(np.searchsorted(rn, i, side="right")) - 1
                pre = np.append(sid[ro[b] + p], t)[None, :]
                assert got[3][i] == trie.node_of(pre)[0]


def pin_full_trie_is_unconstrained(fn, seed=1):
    """Every token sequence an item: every node has all V tokens as
    children, so the selection equals the unconstrained one."""
    rng = np.random.default_rng(seed)
    V, depth = 4, 3
    items = np.array(np.meshgrid(*[np.arange(V)] * depth, indexing="ij")).reshape(depth, -1).T
    trie = I.build_trie(np.ascontiguousarray(items, dtype=np.int32), V)
    for step in range(depth):
        ro = np.array([0, 3, 5]); rn = np.array([0, 7, 10])
        sid = rng.integers(0, V, size=(5, step)).astype(np.int32)
        s = rng.standard_normal(5); x = rng.standard_normal((5, V)) * 2
        got = call(fn, trie, ro, rn, s, x, sid)
        ref = O.beam_select(ro, rn, s, x)
        assert np.array_equal(got[1], ref[1]) and np.array_equal(got[2], ref[2])
        assert np.allclose(got[0], ref[0], atol=1e-12)


def pin_closed_forms(fn):
    """One legal token: its value is the beam's score (probability 1).  All
    of a beam's legal candidates kept: their probabilities sum to 1."""
    V = 7
    items = np.array([[2, 5], [2, 6], [4, 1]], dtype=np.int32)
    trie = I.build_trie(items, V)
    ro = np.array([0, 2]); rn = np.array([0, 5])
    s = np.array([-0.25, -3.0]); x = np.random.default_rng(2).standard_normal((2, V))
    sid = np.array([[4], [2]], dtype=np.int32)        # beam 0: only token 1; beam 1: 5 or 6
    val, p, t, node = call(fn, trie, ro, rn, s, x, sid)
    i0 = [i for i in range(3) if p[i] == 0]
    assert len(i0) == 1 and t[i0[0]] == 1 and val[i0[0]] == -0.25
    i1 = [i for i in range(3) if p[i] == 1]
    assert sorted(t[i] for i in i1) == [5, 6]
    assert abs(sum(math.exp(val[i] + 3.0) for i in i1) - 1.0) < 1e-12
    assert list(p[3:]) == [-1, -1] and np.isinf(val[3:]).all() and list(node[3:]) == [-1, -1]
    # every prefix outside the trie: nothing to keep
    sid = np.array([[3], [0]], dtype=np.int32)
    val, p, t, node = call(fn, trie, ro, rn, s, x, sid)
    assert (p == -1).all() and (t == -1).all() and np.isinf(val).all()
    # a leaf (full item) has no children
    sid = np.array([[2, 5], [4, 1]], dtype=np.int32)
    val, p, t, node = call(fn, trie, ro, rn, s, x, sid)
    assert (p == -1).all()


def pin_shift_invariance(fn, seed=3):
    """Adding a constant to a beam's logits changes nothing."""
    rng = np.random.default_rng(seed)
    items, trie, ro, rn, s, x, sid = tiny_case(rng, step=1)
    a = call(fn, trie, ro, rn, s, x, sid)
    b = call(fn, trie, ro, rn, s, x + rng.standard_normal((x.shape[0], 1)) * 5, sid)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    assert np.allclose(a[0], b[0], atol=1e-12)


def battery(fn):
    failed = []
    for name, pin in (("brute", pin_bruteforce), ("full", pin_full_trie_is_unconstrained),
                      ("closed", pin_closed_forms), ("shift", pin_shift_invariance)):
        try:
            pin(fn)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            failed.append(name)
    return failed


def test_bruteforce():
    pin_bruteforce(O.beam_select_trie)


def test_full_trie_reduces_to_unconstrained():
    pin_full_trie_is_unconstrained(O.beam_select_trie)


def test_closed_forms():
    pin_closed_forms(O.beam_select_trie)


def test_shift_invariance():
    pin_shift_invariance(O.beam_select_trie)


def test_generator_nodes_match_walk():
    """The generator's node ids (prefix lookup) equal the oracle's walk, and
    the CSR holds increasing tokens within each node."""
    trie = I.build_trie(I.sid_catalog(3000, 3, 40, seed=5), 40)
    assert np.all(np.diff(trie.node_ptr) >= 0)
    for u in range(0, trie.n_nodes, 97):
        toks = trie.edge_tok[trie.node_ptr[u]:trie.node_ptr[u + 1]]
        assert np.all(np.diff(toks) > 0)
    ti = I.trie_select_inputs([30, 20], [30, 20], 40, 2, trie, seed=6, dead=0.2)
    for r in range(ti.sid.shape[0]):
        assert ti.node_old[r] == O.trie_walk(trie.node_ptr, trie.edge_tok, trie.edge_child,
                                             ti.sid[r])
    assert (ti.node_old < 0).any()


MUTANTS = [
    ("normalised over the whole vocabulary",
     "lse = m + np.log(np.exp(x - m).sum())",
     "lse = np.log(np.exp(logits[r0 + w]).sum())"),
    ("walk stops one token short",
     "node = trie_walk(node_ptr, edge_tok, edge_child, sid[r0 + w])",
     "node = trie_walk(node_ptr, edge_tok, edge_child, sid[r0 + w][:-1])"),
    ("edge index taken for the token",
     "flats.append(w * V + legal)",
     "flats.append(w * V + np.arange(lo, hi))"),
    ("no constraint: every token legal",
     "legal = np.asarray(edge_tok[lo:hi], dtype=np.int64)",
     "legal = np.arange(V)"),
    ("child of the wrong edge",
     "kids.append(np.asarray(edge_child[lo:hi]))",
     "kids.append(np.asarray(edge_child[lo:hi])[::-1])"),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(name, orig, bad):
    src = textwrap.dedent(inspect.getsource(O.beam_select_trie))
    assert orig in src
    ns = {"np": np, "math": math, "trie_walk": O.trie_walk}
    exec(src.replace(orig, bad, 1), ns)
    assert battery(ns["beam_select_trie"]), f"no pin rejects '{name}'"


WALK_MUTANTS = [
    ("first edge always taken", "hit = np.nonzero(np.asarray(edge_tok[lo:hi]) == int(t))[0]",
     "hit = np.arange(hi - lo)"),
    ("missing token not detected", "        if hit.size == 0:\n            return -1\n",
     "        if hit.size == 0:\n            hit = np.zeros(1, dtype=np.int64)\n"),
]


@pytest.mark.parametrize("name,orig,bad", WALK_MUTANTS, ids=[m[0] for m in WALK_MUTANTS])
def test_walk_mutant_is_rejected(name, orig, bad):
    src = textwrap.dedent(inspect.getsource(O.trie_walk))
    assert orig in src
    ns = {"np": np}
    exec(src.replace(orig, bad, 1), ns)
    sel_src = textwrap.dedent(inspect.getsource(O.beam_select_trie))
    ns2 = {"np": np, "math": math, "trie_walk": ns["trie_walk"]}
    exec(sel_src, ns2)
    assert battery(ns2["beam_select_trie"]), f"no pin rejects '{name}'"


def test_real_oracle_passes_battery():
    assert battery(O.beam_select_trie) == []
