"""GPU parity of item-constrained beam selection (legal next tokens from a
CSR semantic-ID trie, log-softmax over them, top-K over beams) through the C
ABI against the fp64 oracle, which walks every beam's prefix from the root.
Comparison rules as for the unconstrained selection (select_check.py), plus
each kept beam's trie node."""
import numpy as np
import pytest

from gpu_util import log
from oracle import oracle as O
from select_check import check_against_oracle
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu


def run_gpu(ti, K_max):
    import torch
    from shared_prefix_beam_amd import gr_attn
    d = "cuda"
    si, tr = ti.sel, ti.trie

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(d)

    fan = tr.level_fanout(ti.step)                # the step's level bounds every node
    out = gr_attn.beam_select_trie(
        i32(si.row_offset_old), i32(si.row_offset_new), torch.from_numpy(si.score_old).to(d),
        torch.from_numpy(np.ascontiguousarray(si.logits)).to(d), i32(ti.node_old),
        i32(tr.node_ptr), i32(tr.edge_tok), i32(tr.edge_child), K_max, max(fan, 1),
        R_new=int(si.row_offset_new[-1]))
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in out)


def check(ti, K_max, what):
    si, tr = ti.sel, ti.trie
    fan = np.diff(tr.node_ptr)
    per_beam = np.where(ti.node_old >= 0, fan[np.maximum(ti.node_old, 0)], 0)
    ro = si.row_offset_old
    n_cand = np.array([per_beam[ro[b]:ro[b + 1]].sum() for b in range(len(ro) - 1)],
                      dtype=np.int64)
    check_against_oracle(
        si, run_gpu(ti, K_max), K_max, what,
        lambda rw: O.beam_select_trie(ro, rw, si.score_old, si.logits, ti.sid, tr.node_ptr,
                                      tr.edge_tok, tr.edge_child),
        n_cand=n_cand)


@pytest.fixture(scope="module")
def small_trie():
    return I.build_trie(I.sid_catalog(3000, 3, 300, seed=31), 300)


@pytest.mark.parametrize("step", [0, 1, 2, 3])
def test_ragged_steps_with_dead_beams(small_trie, step):
    """Root (every token of the catalog's first level), middle and last
    levels, leaves (no children); ragged requests, some dead beams."""
    ti = I.trie_select_inputs([5, 0, 17, 1, 9], [6, 3, 0, 12, 40], 300, step, small_trie,
                              seed=40 + step, dead=0.2)
    log(f"[trie] ragged step {step}")
    check(ti, 40, f"ragged step {step}")


def test_wide_root_selected_again(small_trie):
    """Two beams at the root (~300 legal tokens, more than a 32-key list) and
    many kept: lists are exhausted above the bound and the rows are selected
    again over their legal tokens."""
    ti = I.trie_select_inputs([2, 3], [200, 64], 300, 0, small_trie, seed=50)
    log("[trie] root rows selected again")
    check(ti, 200, "root reselect")


def test_full_vocabulary_root_matches_unconstrained():
    """A catalog whose first level covers all 8192 tokens: at the root the
    constrained selection is the unconstrained one."""
    tr = I.catalog_trie(**I.TRIE_CATALOG)
    ti = I.trie_select_inputs([64, 40], [64, 40], 8192, 0, tr, seed=51)
    log("[trie] full-vocabulary root")
    gpu = run_gpu(ti, 64)
    si = ti.sel
    ref = O.beam_select(si.row_offset_old, si.row_offset_new, si.score_old, si.logits)
    same = (gpu[1] == ref[1]) & (gpu[2] == ref[2])
    assert same.mean() > 0.99
    assert np.abs(gpu[0][same] - ref[0][same]).max() < 1e-4
    check(ti, 64, "root 8192")


@pytest.mark.parametrize("cfg", sorted(I.TRIE_WORKLOADS))
def test_trie_workloads(cfg):
    """The benchmarked shape: 900 beams x 4 requests, second step (~120
    legal tokens per beam) over the one-million-item catalog."""
    ti = I.trie_workload(cfg)
    log(f"[trie] workload {I.TRIE_WORKLOADS[cfg]['name']}")
    check(ti, int(np.diff(ti.sel.row_offset_new).max()), I.TRIE_WORKLOADS[cfg]["name"])


def test_last_level_few_candidates():
    """Third step of the large catalog: about one legal token per beam, fewer
    candidates than kept beams in a request (padding)."""
    tr = I.catalog_trie(**I.TRIE_CATALOG)
    ti = I.trie_select_inputs([300, 200], [400, 150], 8192, 2, tr, seed=52, dead=0.1)
    log("[trie] last level")
    check(ti, 400, "last level")


def truncated(tr, level, F):
    """CSR copy of trie `tr` whose nodes at `level` keep only their first F
    edges (node ids unchanged): what a call with max_fanout F may consider."""
    lo, hi = int(tr.level_start[level]), int(tr.level_start[level + 1])
    ptr, tok, child = [0], [], []
    for u in range(tr.node_ptr.size - 1):
        a, z = int(tr.node_ptr[u]), int(tr.node_ptr[u + 1])
        if lo <= u < hi:
            z = min(z, a + F)
        tok.extend(tr.edge_tok[a:z].tolist())
        child.extend(tr.edge_child[a:z].tolist())
        ptr.append(len(tok))
    return (np.asarray(ptr, np.int32), np.asarray(tok, np.int32), np.asarray(child, np.int32))


@pytest.mark.parametrize("step", [0, 1])
def test_max_fanout_below_a_node_fanout(small_trie, step):
    """max_fanout below some expanded node's child count: such a node offers
    only its first max_fanout edges (the oracle runs on the trie cut so)."""
    import torch
    from shared_prefix_beam_amd import gr_attn
    tr = small_trie
    F = max(1, tr.level_fanout(step) * 2 // 3)
    ti = I.trie_select_inputs([40, 17, 60], [30, 17, 45], tr.V, step, tr, seed=11 + step, dead=0.1)
    si = ti.sel
    ptr, tok, child = truncated(tr, step, F)
    assert (np.diff(ptr) < np.diff(tr.node_ptr)).any()       # some node is cut
    fan = np.diff(ptr)
    per_beam = np.where(ti.node_old >= 0, fan[np.maximum(ti.node_old, 0)], 0)
    ro = si.row_offset_old
    n_cand = np.array([per_beam[ro[b]:ro[b + 1]].sum() for b in range(len(ro) - 1)], np.int64)
    K_max = int(np.diff(si.row_offset_new).max())

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    log(f"[trie] step {step}: max_fanout {F} below the level's {tr.level_fanout(step)}")
    out = gr_attn.beam_select_trie(
        i32(si.row_offset_old), i32(si.row_offset_new), torch.from_numpy(si.score_old).cuda(),
        torch.from_numpy(np.ascontiguousarray(si.logits)).cuda(), i32(ti.node_old),
        i32(tr.node_ptr), i32(tr.edge_tok), i32(tr.edge_child), K_max, F,
        R_new=int(si.row_offset_new[-1]))
    torch.cuda.synchronize()
    got = tuple(t.cpu().numpy() for t in out)
    check_against_oracle(
        si, got, K_max, f"max_fanout {F} step {step}",
        lambda rw: O.beam_select_trie(ro, rw, si.score_old, si.logits, ti.sid, ptr, tok, child),
        n_cand=n_cand)
