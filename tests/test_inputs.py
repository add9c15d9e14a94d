"""The seeded generator: structure of the synthetic workloads (CPU only)."""
import json
import os

import numpy as np
import pytest

from shared_prefix_beam_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "oracle_golden.json")


@pytest.fixture(scope="module")
def workloads():
    return {i: I.generate(I.WORKLOADS[i]) for i in (1, 2, 3, 4, 5)}


def test_bf16_rounding_is_nearest_even():
    # bf16 keeps 7 fraction bits: one ulp at 1.0 is 2^-7
    u = 2.0 ** -7
    x = np.array([1.0, 1 + u / 2, 1 + 1.5 * u, 1 + 0.75 * u, 1 + 0.25 * u, -2.5], dtype=np.float32)
    exp = np.array([1.0, 1.0, 1 + 2 * u, 1 + u, 1.0, -2.5], dtype=np.float32)  # ties to even
    assert np.array_equal(I.bf16_bits_to_f32(I.to_bf16_bits(x)), exp)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_layout_and_ranges(workloads, cfg):
    inp = workloads[cfg]
    wl = inp.wl
    assert inp.q.shape == (inp.R, wl.Hq, wl.D)
    assert inp.ctx_k.shape == (wl.B, inp.ctx_cap, wl.Hkv, wl.D)
    assert inp.beam_k.shape == (wl.B, inp.T_cap * inp.W_cap + 1, wl.Hkv, wl.D)
    assert inp.R == sum(wl.W)
    assert np.all(inp.ctx_len <= inp.ctx_cap) and np.all(inp.beam_len <= inp.T_cap)
    for b in range(wl.B):
        r0, r1 = inp.row_offset[b], inp.row_offset[b + 1]
        T = int(inp.beam_len[b])
        p = inp.beam_path[r0:r1]
        # valid entries: step s lives in [s*W_cap, s*W_cap + W_s)
        for s in range(T):
            assert np.all(p[:, s] >= s * inp.W_cap)
            assert np.all(p[:, s] < s * inp.W_cap + inp.widths[b][s])
        # the last step is each beam's own slot, except for duplicated rows
        own = np.arange(r1 - r0) + (T - 1) * inp.W_cap
        dup = set(int(x) for x in inp.dup_rows[b])
        for w in range(r1 - r0):
            if T and w not in dup:
                assert p[w, T - 1] == own[w]
        assert np.all(p[:, T:] == inp.T_cap * inp.W_cap)       # padding -> NaN slot


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_padding_is_nan_and_live_data_finite(workloads, cfg):
    inp = workloads[cfg]
    f = lambda a: I.bf16_bits_to_f32(a)
    for b in range(inp.B):
        L = int(inp.ctx_len[b])
        assert np.isfinite(f(inp.ctx_k[b, :L])).all() and np.isnan(f(inp.ctx_k[b, L:])).all()
        assert np.isfinite(f(inp.ctx_v[b, :L])).all() and np.isnan(f(inp.ctx_v[b, L:])).all()
        assert np.isnan(f(inp.beam_k[b, -1])).all()
        r0, r1 = inp.row_offset[b], inp.row_offset[b + 1]
        used = np.unique(inp.beam_path[r0:r1, :int(inp.beam_len[b])])
        assert np.isfinite(f(inp.beam_k[b, used])).all()
        assert np.isfinite(f(inp.beam_v[b, used])).all()
    assert np.isfinite(f(inp.q)).all()


def test_growing_step_widths():
    assert I.step_widths(20, 5, True) == [2, 6, 11, 15, 20]
    assert I.step_widths(900, 5, True) == [112, 309, 506, 703, 900]
    assert I.step_widths(128, 3, False) == [128, 128, 128]
    assert I.step_widths(7, 1, True) == [7]


def test_config5_widths(workloads):
    inp = workloads[5]
    for b, W in enumerate(inp.wl.W):
        assert inp.widths[b] == I.step_widths(W, 5, True)


def test_config4_duplicate_fraction(workloads):
    inp = workloads[4]
    for b in range(inp.B):
        assert len(inp.dup_rows[b]) == 270
        r0 = inp.row_offset[b]
        src = inp.beam_path[r0 + inp.dup_src[b]]
        assert np.all(inp.beam_path[r0 + inp.dup_rows[b]] == src)


def test_config3_ranges(workloads):
    inp = workloads[3]
    assert np.all((inp.ctx_len >= 512) & (inp.ctx_len <= 4096))
    assert np.all((inp.beam_len >= 2) & (inp.beam_len <= 5))
    q = I.bf16_bits_to_f32(inp.q)
    assert 0.45 < q.std() < 0.55


def test_seeds_reproduce_golden_digests(workloads):
    gold = json.load(open(GOLDEN))["input_sha256"]
    for cfg, inp in workloads.items():
        assert inp.digest() == gold[str(cfg)], f"workload {cfg} changed"
