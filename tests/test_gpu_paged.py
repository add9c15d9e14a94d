"""GPU parity of the paged-ContextKV entry point (gr_decode_attn_paged):
against the oracle over the same pages, and bitwise against the dense entry
point on the same data (only the addresses of the context rows differ)."""
import zlib

import numpy as np
import pytest

from gpu_util import assert_parity, log, run_lib
from oracle import oracle as O
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu


def run_paged(inp, pg, tiling=None):
    import torch
    from shared_prefix_beam_amd import gr_attn
    t = I.to_torch(inp)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    out, lse = gr_attn.decode_attn_paged(
        t["q"], bf(pg.k_pages), bf(pg.v_pages),
        torch.from_numpy(pg.page_table.astype(np.int32)).cuda(), pg.page_size, t["ctx_len"],
        t["beam_k"], t["beam_v"], t["beam_path"], t["beam_len"], t["row_offset"],
        W_max=int(max(inp.wl.W)), ctx_cap=inp.ctx_cap, tiling=tiling)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def ragged(D=128, Hq=16, Hkv=8, seed=0):
    return I.custom(B=3, Hq=Hq, Hkv=Hkv, D=D, W=[37, 5, 70], ctx_len=[1000, 33, 517],
                    beam_len=[3, 1, 5], seed=seed)


@pytest.mark.parametrize("page_size", [16, 32, 48, 64, 80, 128])
def test_paged_ragged_all_rows(page_size):
    inp = ragged(seed=page_size)
    pg = I.to_paged(inp, page_size, seed=page_size + 1)
    log(f"[paged] ragged page_size={page_size} R={inp.R}")
    out, lse = run_paged(inp, pg)
    ref_out, ref_lse = O.decode_attn_paged(inp.q, pg.k_pages, pg.v_pages, pg.page_table,
                                           page_size, inp.ctx_len, inp.beam_k, inp.beam_v,
                                           inp.beam_path, inp.beam_len, inp.row_offset,
                                           ctx_cap=inp.ctx_cap, scale=inp.scale)
    assert_parity(out, lse, ref_out, ref_lse, f"paged {page_size}")
    dense_out, dense_lse = run_lib(inp, "fused")
    assert np.array_equal(out, dense_out) and np.array_equal(lse, dense_lse), \
        "paged and dense results differ"


@pytest.mark.parametrize("Hq,Hkv", [(8, 4), (16, 4), (16, 2)], ids=["g2", "g4", "g8"])
def test_paged_d64(Hq, Hkv):
    inp = ragged(D=64, Hq=Hq, Hkv=Hkv, seed=64 + Hq + Hkv)
    pg = I.to_paged(inp, 16, seed=65)
    log(f"[paged] D=64 G={Hq // Hkv} page 16 R={inp.R}")
    out, lse = run_paged(inp, pg)
    ref_out, ref_lse = O.decode_attn_paged(inp.q, pg.k_pages, pg.v_pages, pg.page_table, 16,
                                           inp.ctx_len, inp.beam_k, inp.beam_v, inp.beam_path,
                                           inp.beam_len, inp.row_offset, ctx_cap=inp.ctx_cap,
                                           scale=inp.scale)
    assert_parity(out, lse, ref_out, ref_lse, f"paged d64 g{Hq // Hkv}")
    dense_out, dense_lse = run_lib(inp, "fused")
    assert np.array_equal(out, dense_out) and np.array_equal(lse, dense_lse)


TILINGS = [(128, 8, 1), (128, 4, 1), (128, 4, 2), (128, 2, 2), (64, 4, 1), (64, 2, 2), (64, 2, 4)]


@pytest.mark.parametrize("page_size", [16, 48], ids=["p16", "p48"])
@pytest.mark.parametrize("split", [1, 3], ids=["s1", "s3"])
@pytest.mark.parametrize("tiling", TILINGS, ids=[f"d{d}_q{a}_k{c}" for d, a, c in TILINGS])
def test_paged_every_tiling(tiling, split, page_size):
    D, nqt, nks = tiling
    inp = ragged(D=D, Hq=16 if D == 128 else 8, Hkv=8 if D == 128 else 4, seed=nqt * 7 + nks)
    pg = I.to_paged(inp, page_size, seed=3)
    log(f"[paged] tiling {tiling} split {split} page {page_size}")
    out, lse = run_paged(inp, pg, tiling=(nqt, nks, split))
    dense_out, dense_lse = run_lib(inp, "fused", tiling=(nqt, nks, split))
    assert np.array_equal(out, dense_out) and np.array_equal(lse, dense_lse)


TILINGS16 = [(128, 4, 2), (128, 8, 1), (128, 4, 1), (128, 6, 1), (128, 2, 2), (64, 4, 2),
             (64, 8, 1)]


@pytest.mark.parametrize("page_size", [16, 48], ids=["p16", "p48"])
@pytest.mark.parametrize("tiling", [(4, 2, 1, True), (4, 1, 1, False)], ids=["row16_q4_k2", "q4_k1"])
def test_paged_long_context(tiling, page_size):
    """A 17k-token context over more than a thousand pages, with a page size
    that is a power of two (shift and mask) and one that is not (division):
    bitwise equal to the dense launch."""
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[9, 40], ctx_len=[16993, 700],
                   beam_len=[2, 3], seed=77)
    pg = I.to_paged(inp, page_size, seed=78)
    assert pg.page_table.shape[1] * page_size >= 16993
    log(f"[paged] long context, {pg.page_table.shape[1]} pages of {page_size}, tiling {tiling}")
    out, lse = run_paged(inp, pg, tiling=tiling)
    dense_out, dense_lse = run_lib(inp, "fused", tiling=tiling)
    assert np.array_equal(out, dense_out) and np.array_equal(lse, dense_lse)


@pytest.mark.parametrize("page_size", [16, 48], ids=["p16", "p48"])
@pytest.mark.parametrize("tiling", TILINGS16, ids=[f"d{d}_q{a}_k{c}" for d, a, c in TILINGS16])
def test_paged_row16_tilings(tiling, page_size):
    """16-row waves on a paged context: bitwise equal to the dense launch."""
    D, nqt, nks = tiling
    inp = ragged(D=D, Hq=16 if D == 128 else 8, Hkv=8 if D == 128 else 4, seed=nqt * 5 + nks)
    pg = I.to_paged(inp, page_size, seed=4)
    log(f"[paged] row16 tiling {tiling} page {page_size}")
    out, lse = run_paged(inp, pg, tiling=(nqt, nks, 1, True))
    dense_out, dense_lse = run_lib(inp, "fused", tiling=(nqt, nks, 1, True))
    assert np.array_equal(out, dense_out) and np.array_equal(lse, dense_lse)


@pytest.mark.parametrize("cfg,page_size", [(2, 16), (4, 64), (3, 32)])
def test_paged_workloads(cfg, page_size):
    inp = I.generate(I.WORKLOADS[cfg])
    pg = I.to_paged(inp, page_size, seed=cfg)
    log(f"[paged] workload {cfg} page {page_size} R={inp.R}")
    out, lse = run_paged(inp, pg)
    ref_out, ref_lse = O.decode_attn_paged(inp.q, pg.k_pages, pg.v_pages, pg.page_table,
                                           page_size, inp.ctx_len, inp.beam_k, inp.beam_v,
                                           inp.beam_path, inp.beam_len, inp.row_offset,
                                           ctx_cap=inp.ctx_cap, scale=inp.scale)
    assert np.isfinite(out).all()
    assert_parity(out, lse, ref_out, ref_lse, f"paged cfg{cfg}")


@pytest.mark.parametrize("page_size", [16, 48], ids=["p16", "p48"])
@pytest.mark.parametrize("tiling", [(4, 1, 1, False), (4, 1, 3, False), (4, 2, 1, True)],
                         ids=["q4_k1", "q4_k1_s3", "row16_q4_k2"])
def test_paged_rising_scores_take_exact_sweep(tiling, page_size):
    """Scores that grow by far more than 44 nats along the context: the exact
    re-sweep runs, and reads the pages a second time through the table."""
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[40, 7], ctx_len=[600, 250], beam_len=[2, 3],
                   seed=9)
    k = I.bf16_bits_to_f32(inp.ctx_k).copy()
    ramp = np.linspace(0.05, 6.0, inp.ctx_cap, dtype=np.float32)[None, :, None, None]
    inp.ctx_k[:] = I.to_bf16_bits(k * ramp)
    inp.q[:] = I.to_bf16_bits(I.bf16_bits_to_f32(inp.q) * np.float32(4.0))
    pg = I.to_paged(inp, page_size, seed=10)
    log(f"[paged] rising scores (exact re-sweep) page {page_size} tiling {tiling}")
    out, lse = run_paged(inp, pg, tiling=tiling)
    ref_out, ref_lse = O.decode_attn_paged(inp.q, pg.k_pages, pg.v_pages, pg.page_table,
                                           page_size, inp.ctx_len, inp.beam_k, inp.beam_v,
                                           inp.beam_path, inp.beam_len, inp.row_offset,
                                           ctx_cap=inp.ctx_cap, scale=inp.scale)
    assert (ref_lse > 60).any()
    assert_parity(out, lse, ref_out, ref_lse, f"paged rising {page_size} {tiling}")
    dense_out, dense_lse = run_lib(inp, "fused", tiling=tiling)
    assert np.array_equal(out, dense_out) and np.array_equal(lse, dense_lse)
