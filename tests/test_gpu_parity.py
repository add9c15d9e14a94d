"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: max abs 2e-2 and row-wise max rel 1e-2 on bf16 outputs, 1e-3 abs
on fp32 LSE.
"""
import zlib

import numpy as np
import pytest

from gpu_util import assert_parity, log, run_lib
from oracle import oracle as O
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu

_cache = {}
_ref = {}


def workload(cfg):
    if cfg not in _cache:
        _cache[cfg] = I.generate(I.WORKLOADS[cfg])
    return _cache[cfg]


def workload_ref(cfg):
    """The oracle's result on every row of the workload (computed once)."""
    if cfg not in _ref:
        _ref[cfg] = O.decode_attn_inputs(workload(cfg))
    return _ref[cfg]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("which", ["fused", "generic"])
def test_workload_parity(cfg, which):
    """Full-size workloads, in the launch configuration the benchmark times:
    every output row and head against the fp64 oracle."""
    inp = workload(cfg)
    log(f"[parity] workload {cfg} ({inp.wl.name}) path={which} R={inp.R}")
    out, lse = run_lib(inp, which)
    ref_out, ref_lse = workload_ref(cfg)
    assert np.isfinite(out).all(), "NaN/inf anywhere in the output"
    assert_parity(out, lse, ref_out, ref_lse, f"cfg{cfg}/{which}")


SMALL = [
    # (name, B, Hq, Hkv, D, W, ctx_len, beam_len, kwargs)
    ("ragged_tails", 3, 16, 8, 128, [37, 5, 70], [1000, 33, 517], [3, 1, 5], {}),
    ("g4_growing", 2, 32, 8, 128, [20, 45], [700, 1300], [5, 4], dict(grow_steps=True)),
    ("d64_g2", 2, 4, 2, 64, [9, 40], [95, 300], [2, 3], {}),
    ("mha_g1", 2, 8, 8, 128, [33, 64], [129, 64], [2, 2], {}),
    ("g8", 1, 8, 1, 128, [24], [250], [3], {}),
    ("one_beam", 2, 16, 8, 128, [1, 1], [513, 2], [3, 1], {}),
    ("ctx_len_1", 2, 16, 8, 128, [4, 7], [1, 1], [2, 3], {}),
    ("no_beam_tokens", 2, 16, 8, 128, [6, 3], [300, 77], [0, 0], dict(T_cap=3)),
    ("no_context", 2, 16, 8, 128, [6, 3], [0, 0], [3, 2], dict(ctx_cap=64)),
    ("empty_request", 3, 16, 8, 128, [5, 0, 4], [64, 50, 0], [2, 2, 0], dict(ctx_cap=64)),
    ("no_keys_at_all", 1, 16, 8, 128, [3], [0], [0], dict(ctx_cap=32, T_cap=2)),
    ("dup_paths", 2, 16, 8, 128, [60, 40], [256, 130], [3, 3], dict(dup_frac=0.3)),
    ("sharp_q8", 2, 16, 8, 128, [30, 20], [900, 400], [3, 4], dict(q_std=8.0)),
    # group sizes that do not divide a wave's 32 query columns: per-lane gathers
    ("g3", 2, 24, 8, 128, [30, 11], [700, 65], [3, 2], {}),
    ("g5", 2, 40, 8, 128, [13, 7], [300, 90], [4, 1], {}),
    ("g6", 2, 48, 8, 128, [22, 9], [500, 120], [3, 5], {}),
    ("g7", 1, 56, 8, 128, [10], [260], [3], {}),
    # D = 64 at the larger groups (G = 8: fewer beams per wave than rows per load)
    ("d64_g4", 2, 16, 4, 64, [21, 40], [300, 97], [3, 2], {}),
    ("d64_g8", 2, 16, 2, 64, [17, 40], [333, 64], [3, 4], {}),
    ("d64_g8_mha_heads", 1, 64, 8, 64, [12], [150], [5], {}),
    # few beams against long contexts: the planner splits each pair's context
    # over several workgroups (partials combined through the workspace)
    ("long_ctx_few_beams", 1, 16, 8, 128, [4], [8000], [3], {}),
    ("long_ctx_g4", 2, 32, 8, 128, [3, 5], [6000, 3000], [5, 2], {}),
    # BeamPath tables larger than the staged 4 KB (entries loaded per lane)
    ("ptab_overflow_g1", 1, 8, 8, 128, [150], [300], [9], {}),
    ("ptab_overflow_g2", 2, 16, 8, 128, [100, 64], [200, 129], [17, 12], {}),
    # one very wide request: 2048 beams x 8 query heads = 16384 stacked rows
    # on a single (request, KV head) pair (128 query tiles of one pair)
    ("wide_2048_beams_g8", 1, 8, 1, 128, [2048], [200], [3], dict(dup_frac=0.3)),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("which", ["fused", "generic"])
def test_small_shapes_all_rows(case, which):
    name, B, Hq, Hkv, D, W, L, T, kw = case
    inp = I.custom(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, ctx_len=L, beam_len=T, seed=zlib.crc32(name.encode()) % 1000,
                   **kw)
    log(f"[parity] {name} path={which} R={inp.R} L={L} T={T}")
    out, lse = run_lib(inp, which)
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"{name}/{which}")


def test_long_context_all_rows():
    """A 131,072-token context shared by six beams, beside a short request:
    the planner splits each pair's context over eight workgroups of 512
    tiles each.  Every row against the oracle (fused path only: the generic
    comparator is limited to 16,384 keys)."""
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[6, 3], ctx_len=[131072, 100], beam_len=[3, 2],
                   seed=4242)
    log(f"[parity] long context L={inp.ctx_len.tolist()} R={inp.R}")
    out, lse = run_lib(inp, "fused")
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, "long context")


TILINGS = [(128, 8, 1), (128, 4, 1), (128, 4, 2), (128, 2, 2), (64, 4, 1), (64, 2, 2), (64, 2, 4)]
SPLITS = [1, 2, 3, 8]


@pytest.mark.parametrize("split", SPLITS, ids=[f"s{s}" for s in SPLITS])
@pytest.mark.parametrize("tiling", TILINGS, ids=[f"d{d}_q{a}_k{c}" for d, a, c in TILINGS])
def test_every_tiling_ragged(tiling, split):
    """Each compiled (query tile, key streams) shape with the context split
    over 1, 2, 3 and 8 workgroups, forced per call, on ragged requests:
    partial context tiles, partial query tiles, streams and splits with
    unequal tile counts, empty ones (the 33-token context has 2 tiles) and
    beam steps spread over the streams of several workgroups."""
    D, nqt, nks = tiling
    Hq, Hkv = (16, 8) if D == 128 else (8, 4)
    inp = I.custom(B=3, Hq=Hq, Hkv=Hkv, D=D, W=[37, 5, 130], ctx_len=[1000, 33, 517],
                   beam_len=[3, 1, 5], seed=100 + nqt * 10 + nks + 1000 * split)
    log(f"[parity] tiling D={D} NQT={nqt} NKS={nks} split={split} R={inp.R}")
    out, lse = run_lib(inp, "fused", tiling=(nqt, nks, split))
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"tiling {tiling} split {split}")


TILINGS16 = [(128, 4, 2), (128, 8, 1), (128, 4, 1), (128, 6, 1), (128, 2, 2), (64, 4, 2),
             (64, 8, 1)]


@pytest.mark.parametrize("tiling", TILINGS16, ids=[f"d{d}_q{a}_k{c}" for d, a, c in TILINGS16])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_row16_tilings_ragged(tiling, G):
    """Waves of 16 stacked query rows (the 16x16x32 kernel), each compiled
    tiling forced per call, on ragged requests with every group size."""
    D, nqt, nks = tiling
    Hkv = 8 if G <= 4 else 2
    inp = I.custom(B=3, Hq=Hkv * G, Hkv=Hkv, D=D, W=[37, 5, 70], ctx_len=[1000, 33, 517],
                   beam_len=[3, 1, 5], seed=200 + nqt * 10 + nks + 1000 * G)
    log(f"[parity] row16 D={D} NQT={nqt} NKS={nks} G={G} R={inp.R}")
    out, lse = run_lib(inp, "fused", tiling=(nqt, nks, 1, True))
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"row16 {tiling} G={G}")


@pytest.mark.parametrize("tiling", TILINGS, ids=[f"d{d}_q{a}_k{c}" for d, a, c in TILINGS])
def test_many_steps_short_context(tiling):
    """The 32-row kernel with more BeamKV steps than its gather area holds at
    once (chunks of steps) against contexts of zero to two tiles."""
    D, nqt, nks = tiling
    Hq, Hkv = (16, 8) if D == 128 else (8, 4)
    inp = I.custom(B=3, Hq=Hq, Hkv=Hkv, D=D, W=[37, 5, 20], ctx_len=[0, 33, 64],
                   beam_len=[17, 9, 17], seed=400 + nqt * 10 + nks + D)
    log(f"[parity] many steps D={D} NQT={nqt} NKS={nks} R={inp.R}")
    out, lse = run_lib(inp, "fused", tiling=(nqt, nks, 1))
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"many steps {tiling}")


@pytest.mark.parametrize("tiling", TILINGS16, ids=[f"d{d}_q{a}_k{c}" for d, a, c in TILINGS16])
def test_row16_many_steps_short_context(tiling):
    """More BeamKV steps than the sweep has barriers (contexts of zero to two
    tiles against 9 and 17 path tokens): beam waves fold the remaining steps
    after the sweep's last barrier, sweep waves fold theirs before it."""
    D, nqt, nks = tiling
    Hq, Hkv = (16, 8) if D == 128 else (8, 4)
    inp = I.custom(B=3, Hq=Hq, Hkv=Hkv, D=D, W=[37, 5, 20], ctx_len=[0, 33, 64],
                   beam_len=[17, 9, 17], seed=300 + nqt * 10 + nks + D)
    log(f"[parity] row16 many steps D={D} NQT={nqt} NKS={nks} R={inp.R}")
    out, lse = run_lib(inp, "fused", tiling=(nqt, nks, 1, True))
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"row16 many steps {tiling}")


@pytest.mark.parametrize("cfg,tiling", [(2, (4, 2)), (4, (6, 1)), (4, (8, 1)), (3, (6, 1)),
                                        (5, (6, 1))])
def test_row16_workloads(cfg, tiling):
    """Full workloads through the 16-row kernel: every row against the oracle."""
    inp = workload(cfg)
    log(f"[parity] row16 workload {cfg} tiling {tiling}")
    out, lse = run_lib(inp, "fused", tiling=(tiling[0], tiling[1], 1, True))
    ref_out, ref_lse = workload_ref(cfg)
    assert_parity(out, lse, ref_out, ref_lse, f"row16 cfg{cfg} {tiling}")


def test_row16_rising_scores_take_exact_sweep():
    inp = I.custom(B=1, Hq=16, Hkv=8, D=128, W=[40], ctx_len=[600], beam_len=[2], seed=9)
    k = I.bf16_bits_to_f32(inp.ctx_k).copy()
    ramp = np.linspace(0.05, 6.0, inp.ctx_cap, dtype=np.float32)[None, :, None, None]
    inp.ctx_k[:] = I.to_bf16_bits(k * ramp)
    inp.q[:] = I.to_bf16_bits(I.bf16_bits_to_f32(inp.q) * np.float32(4.0))
    log("[parity] row16 rising scores (exact re-sweep)")
    out, lse = run_lib(inp, "fused", tiling=(4, 2, 1, True))
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert (ref_lse > 60).any()
    assert_parity(out, lse, ref_out, ref_lse, "row16 rising")


def test_split_is_deterministic():
    """The last workgroup of a split unit combines the partials in ascending
    split order whichever workgroup it is: repeated calls are bitwise equal."""
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[64, 33], ctx_len=[2000, 700],
                   beam_len=[3, 2], seed=77)
    log("[parity] split determinism")
    a = run_lib(inp, "fused", tiling=(4, 1, 8))
    for _ in range(3):
        b = run_lib(inp, "fused", tiling=(4, 1, 8))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def rising_inputs(D=128, Hq=16, Hkv=8, W=(40,), ctx_len=(600,), beam_len=(2,), q_mult=4.0):
    """Scores that grow by far more than 44 nats along the context: a
    workgroup whose sweep starts at the first tile overflows its fixed
    first-tile reference, so the exact re-sweep (max pass, then accumulation)
    must run."""
    inp = I.custom(B=len(W), Hq=Hq, Hkv=Hkv, D=D, W=list(W), ctx_len=list(ctx_len),
                   beam_len=list(beam_len), seed=9)
    k = I.bf16_bits_to_f32(inp.ctx_k).copy()
    ramp = np.linspace(0.05, 6.0, inp.ctx_cap, dtype=np.float32)[None, :, None, None]
    k = k * ramp
    q = I.bf16_bits_to_f32(inp.q) * np.float32(q_mult)
    inp.ctx_k[:] = I.to_bf16_bits(k)
    inp.q[:] = I.to_bf16_bits(q)
    # some (row, head) of request 0 has its context maximum more than 64
    # (log2 units) above its first tile's: fixed-reference sums cannot hold it
    G = Hq // Hkv
    n0 = int(inp.row_offset[1])
    qq = I.bf16_bits_to_f32(inp.q)[:n0].astype(np.float64)
    kk = I.bf16_bits_to_f32(inp.ctx_k)[0, :int(inp.ctx_len[0])].astype(np.float64)
    sc = np.einsum("rhd,lhd->rhl", qq, np.repeat(kk, G, axis=1)) * inp.scale / np.log(2.0)
    assert (sc.max(axis=2) - sc[:, :, :32].max(axis=2)).max() > 64
    return inp


@pytest.mark.parametrize("tiling", [None, (4, 1, 1), (8, 1, 1), (4, 2, 1), (2, 2, 1), (4, 1, 2)],
                         ids=["planner", "q4_k1", "q8_k1", "q4_k2", "q2_k2", "q4_k1_s2"])
def test_rising_scores_take_exact_sweep(tiling):
    inp = rising_inputs()
    log(f"[parity] rising scores (exact re-sweep) tiling {tiling}")
    out, lse = run_lib(inp, tiling=tiling)
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert (ref_lse > 60).any()
    assert_parity(out, lse, ref_out, ref_lse, f"rising {tiling}")


RISING_MORE = [
    # (name, D, Hq, Hkv, tiling)
    ("d64_q4_k1", 64, 8, 4, (4, 1, 1)),
    ("d64_q2_k2", 64, 8, 4, (2, 2, 1)),
    ("d64_q2_k4", 64, 8, 4, (2, 4, 1)),
    ("d64_planner", 64, 8, 4, None),
    ("g3_q4_k1", 128, 24, 8, (4, 1, 1)),
    ("g3_planner", 128, 24, 8, None),
    ("g8_q4_k1", 128, 8, 1, (4, 1, 1)),
]


@pytest.mark.parametrize("case", RISING_MORE, ids=[c[0] for c in RISING_MORE])
def test_rising_scores_more_shapes(case):
    """The exact re-sweep at D = 64, with per-lane BeamKV gathers (G = 3) and
    at G = 8, on two ragged requests (the second with a short context)."""
    name, D, Hq, Hkv, tiling = case
    inp = rising_inputs(D=D, Hq=Hq, Hkv=Hkv, W=(40, 7), ctx_len=(600, 250), beam_len=(2, 3),
                        q_mult=4.0 if D == 128 else 6.0)
    log(f"[parity] rising scores {name} tiling {tiling}")
    out, lse = run_lib(inp, tiling=tiling)
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"rising {name}")


@pytest.mark.parametrize("tiling", TILINGS16, ids=[f"d{d}_q{a}_k{c}" for d, a, c in TILINGS16])
def test_row16_rising_every_tiling(tiling):
    """The 16-row kernel's exact re-sweep (its own max-only pass) on every
    compiled 16-row tiling, with and without beam waves."""
    D, nqt, nks = tiling
    inp = rising_inputs(D=D, Hq=16 if D == 128 else 8, Hkv=8 if D == 128 else 4, W=(40, 7),
                        ctx_len=(600, 250), beam_len=(2, 3), q_mult=4.0 if D == 128 else 6.0)
    log(f"[parity] row16 rising scores tiling {tiling}")
    out, lse = run_lib(inp, "fused", tiling=(nqt, nks, 1, True))
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"row16 rising {tiling}")


def test_beam_dominant_and_context_dominant_rows():
    """The BeamKV partial, folded before the context sweep, seeds the
    accumulators after a rescale to the sweep's reference.  Request 0: each
    beam's current token has K = 3 q for the group's first head, so that
    head's beam scores exceed every context score by tens of nats (the
    reference is the beam maximum).  Request 1: beam keys -3 q, scores far
    below the context (the beam partial is rescaled by a tiny factor)."""
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[40, 20], ctx_len=[700, 300], beam_len=[3, 2],
                   seed=31)
    G = inp.wl.Hq // inp.wl.Hkv
    q = I.bf16_bits_to_f32(inp.q)
    bk = I.bf16_bits_to_f32(inp.beam_k).copy()
    for b, sign in ((0, 3.0), (1, -3.0)):
        T = int(inp.beam_len[b])
        for r in range(int(inp.row_offset[b]), int(inp.row_offset[b + 1])):
            for s in range(T):
                p = int(inp.beam_path[r, s])
                if b == 0 and s < T - 1:
                    continue                       # request 0: only the current token
                for g in range(inp.wl.Hkv):
                    bk[b, p, g, :] = sign * q[r, g * G, :]
    inp.beam_k[:] = I.to_bf16_bits(bk)
    log("[parity] beam-dominant and context-dominant rows")
    out, lse = run_lib(inp)
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, "beam/context dominance")


def test_explicit_scale():
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[10, 7], ctx_len=[200, 90], beam_len=[3, 2],
                   seed=17)
    log("[parity] explicit scale 0.05")
    out, lse = run_lib(inp, scale=0.05)
    ref_out, ref_lse = O.decode_attn(
        inp.q, inp.ctx_k, inp.ctx_v, inp.ctx_len, inp.beam_k, inp.beam_v, inp.beam_path,
        inp.beam_len, inp.row_offset, scale=0.05)
    assert_parity(out, lse, ref_out, ref_lse, "scale0.05")


@pytest.mark.parametrize("tiling", [None, (4, 1, 1), (4, 2, 1, True)], ids=["planner", "q4_k1", "row16"])
def test_many_small_requests(tiling):
    """129 requests of 0-6 beams (1032 (request, KV head) pairs, not a
    multiple of the 8 XCDs), contexts of 0-300 tokens and 0-4 path tokens:
    every row against the oracle, and paged bitwise equal to dense."""
    from test_gpu_paged import run_paged
    rng = np.random.default_rng(129)
    B = 129
    W = [int(x) for x in rng.integers(0, 7, size=B)]
    L = [int(x) for x in rng.integers(0, 301, size=B)]
    T = [int(x) for x in rng.integers(0, 5, size=B)]
    inp = I.custom(B=B, Hq=16, Hkv=8, D=128, W=W, ctx_len=L, beam_len=T, seed=129)
    log(f"[parity] many small requests B={B} R={inp.R} tiling {tiling}")
    out, lse = run_lib(inp, "fused", tiling=tiling)
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"many requests {tiling}")
    pg = I.to_paged(inp, 32, seed=130)
    p_out, p_lse = run_paged(inp, pg, tiling=tiling)
    assert np.array_equal(p_out, out) and np.array_equal(p_lse, lse), "paged and dense differ"
