"""The fp64 oracle against facts it does not compute itself (CPU only)."""
import numpy as np
import pytest

import pins
from oracle import oracle as O
from shared_prefix_beam_amd import inputs as I

fn = O.decode_attn


@pytest.fixture(scope="module")
def workloads():
    return {i: I.generate(I.WORKLOADS[i]) for i in (1, 2, 3, 4, 5)}


def sample_rows(inp, n, seed=0):
    """First and last row of every request plus random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(inp.B):
        rows.add(int(inp.row_offset[b]))
        rows.add(int(inp.row_offset[b + 1]) - 1)
    rows.update(int(x) for x in rng.integers(0, inp.R, size=n))
    return sorted(rows)


def test_s1_plain_attention():
    pins.pin_s1_plain_attention(fn)
    pins.pin_s1_plain_attention(fn, seed=8)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_s2_concatenation_workloads(workloads, cfg):
    inp = workloads[cfg]
    rows = range(inp.R) if cfg == 1 else sample_rows(inp, 4, seed=cfg)
    pins.pin_s2_concatenation(fn, inp, rows)


def test_s2_ragged_and_growing():
    for seed in range(3):
        inp = I.custom(B=3, Hq=6, Hkv=3, D=24, W=[5, 1, 7], ctx_len=[0, 13, 30],
                       beam_len=[4, 0, 2], seed=40 + seed, ctx_cap=32, T_cap=5,
                       grow_steps=True)
        pins.pin_s2_concatenation(fn, inp, range(inp.R))


def test_s3_bruteforce_tiny():
    for c in pins.tiny_cases(8):
        pins.pin_s3_bruteforce(fn, c)


def test_s3_bruteforce_sharp_softmax():
    pins.pin_s3_bruteforce(fn, pins.sharp_case())
    pins.pin_s3_bruteforce(fn, pins.sharp_case(seed=32))


def test_s3_bruteforce_config1(workloads):
    pins.pin_s3_bruteforce(fn, workloads[1], rows=[0, 3])


def test_s4_closed_forms():
    pins.pin_s4_closed_forms(fn)


def test_s5_permutation(workloads):
    pins.pin_s5_permutation(fn, workloads[1])
    inp = I.custom(B=3, Hq=4, Hkv=2, D=32, W=[8, 3, 5], ctx_len=[20, 50, 9],
                   beam_len=[3, 1, 2], seed=55)
    pins.pin_s5_permutation(fn, inp)


def test_s6_duplicates_config4_shape():
    # the 30%-duplicate-path recipe at a reduced size (full size is a GPU case)
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[40, 30], ctx_len=[64, 48],
                   beam_len=[3, 3], seed=404, dup_frac=0.3)
    pins.pin_s6_duplicates(fn, inp)


def test_s7_lse_merge(workloads):
    pins.pin_s7_lse_merge(fn, workloads[1], range(4))
    inp = I.custom(B=2, Hq=4, Hkv=1, D=64, W=[4, 6], ctx_len=[100, 3], beam_len=[5, 2],
                   seed=77, grow_steps=True)
    pins.pin_s7_lse_merge(fn, inp, range(inp.R))


def test_s8_gqa():
    pins.pin_s8_gqa(fn)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_nan_padding_never_leaks(workloads, cfg):
    inp = workloads[cfg]
    rows = None if cfg in (1, 2) else sample_rows(inp, 16, seed=cfg)
    pins.pin_nan_padding(fn, inp, rows=rows)


def test_thread_count_does_not_change_results(workloads):
    inp = workloads[2]
    rows = sample_rows(inp, 24)
    a = O.decode_attn_inputs(inp, rows=rows, n_threads=1)
    b = O.decode_attn_inputs(inp, rows=rows, n_threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rows_subset_matches_full(workloads):
    inp = workloads[1]
    full = O.decode_attn_inputs(inp)
    part = O.decode_attn_inputs(inp, rows=[3, 1])
    assert np.array_equal(part[0], full[0][[3, 1]])


def test_bad_arguments_rejected():
    inp = I.generate(I.WORKLOADS[1])
    with pytest.raises(RuntimeError):
        O.decode_attn(inp.q, inp.ctx_k, inp.ctx_v, inp.ctx_len, inp.beam_k, inp.beam_v,
                      inp.beam_path, inp.beam_len, inp.row_offset, rows=[inp.R + 5])


def test_oracle_matches_its_recorded_outputs(workloads):
    """Regression guard: the oracle's own outputs recorded by
    tests/golden/make_golden.py (any change to its arithmetic shows here)."""
    import json, os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "oracle_golden.json")))["oracle"]
    for cfg in ("1", "2"):
        g = gold[cfg]
        out, lse = O.decode_attn_inputs(workloads[int(cfg)], rows=g["rows"])
        assert np.max(np.abs(out - np.array(g["out"]))) < 1e-14
        assert np.max(np.abs(lse - np.array(g["lse"]))) < 1e-14
