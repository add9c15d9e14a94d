"""gr_decode_attn_noalloc (the split's counters and partials in the library's
own device scratch, nothing allocated) through the C ABI, against
gr_decode_attn with a caller-owned workspace on the same inputs: two calls
in a row, the second with a smaller input, with and without a context
split.  The results must be bitwise equal (same kernels, same plan, a fixed
merge order) and within the parity tolerances of the fp64 oracle."""
import numpy as np
import pytest

from gpu_util import assert_parity, log
from oracle import oracle as O
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu


def run_both(inp, tiling=None):
    import torch
    from shared_prefix_beam_amd import gr_attn
    t = I.to_torch(inp)
    W_max = int(max(inp.wl.W))
    stream = torch.cuda.current_stream()
    # existing entry point, caller-owned workspace
    ref_out, ref_lse = gr_attn.decode_attn(t["q"], t["ctx_k"], t["ctx_v"], t["ctx_len"],
                                           t["beam_k"], t["beam_v"], t["beam_path"],
                                           t["beam_len"], t["row_offset"], W_max=W_max,
                                           tiling=tiling)
    # no-alloc entry point through the C ABI: the dims carry no workspace
    dims = gr_attn.make_dims(t["q"], t["ctx_k"], t["beam_k"], t["beam_path"], W_max,
                             tiling=tiling)
    split = gr_attn.gr_decode_attn_workspace_bytes(dims) > 0
    out = torch.full_like(t["q"], float("nan"))
    lse = torch.full(t["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    st = gr_attn.gr_decode_attn_noalloc(
        dims, t["row_offset"].data_ptr(), t["q"].data_ptr(), t["ctx_k"].data_ptr(),
        t["ctx_v"].data_ptr(), t["ctx_len"].data_ptr(), t["beam_k"].data_ptr(),
        t["beam_v"].data_ptr(), t["beam_path"].data_ptr(), t["beam_len"].data_ptr(),
        out.data_ptr(), lse.data_ptr(), stream.cuda_stream)
    assert st == gr_attn.GR_OK, gr_attn.gr_status_str(st)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), lse.cpu().numpy(), ref_out.float().cpu().numpy(),
            ref_lse.cpu().numpy(), split)


CASES = [
    # (name, B, Hq, Hkv, W, ctx_len, beam_len, tiling)
    ("forced_split8", 2, 16, 8, [37, 5], [1000, 33], [3, 1], (4, 1, 8)),
    ("planned_split", 1, 16, 8, [4], [8000], [3], None),
    ("smaller_split3", 2, 16, 8, [9, 3], [300, 77], [2, 3], (4, 1, 3)),
    ("no_split", 2, 16, 8, [20, 9], [300, 77], [2, 3], None),
]


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_matches_workspace_entry_point(order):
    cases = CASES if order == "large_then_small" else CASES[::-1]
    for name, B, Hq, Hkv, W, L, T, tiling in cases:
        inp = I.custom(B=B, Hq=Hq, Hkv=Hkv, D=128, W=W, ctx_len=L, beam_len=T,
                       seed=sum(map(ord, name)))
        log(f"[noalloc] {order} {name} R={inp.R} tiling={tiling}")
        out, lse, ref_out, ref_lse, split = run_both(inp, tiling)
        assert split == (name != "no_split")
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse), name
        o_out, o_lse = O.decode_attn_inputs(inp)
        assert_parity(out, lse, o_out, o_lse, f"noalloc {name}")


def test_noalloc_random_shapes_in_a_row():
    """The seeded random shapes of test_gpu_random.py, one after another
    through both entry points (the scratch keeps each call's leftovers):
    bitwise equal where the split fits the library's scratch, refused with
    GR_ERR_WORKSPACE exactly where it does not (counters beyond 64 KB or
    partials beyond the rest of the 16 MB)."""
    import torch
    from shared_prefix_beam_amd import gr_attn
    from test_gpu_random import N_CASES, draw
    scratch, counters = 16 << 20, 64 << 10
    n_run = 0
    for seed in range(N_CASES):
        D, Hq, Hkv, B, W, L, T, kw = draw(seed)
        inp = I.custom(B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, ctx_len=L, beam_len=T, seed=seed, **kw)
        t = I.to_torch(inp)
        W_max = int(max(inp.wl.W))
        dims = gr_attn.make_dims(t["q"], t["ctx_k"], t["beam_k"], t["beam_path"], W_max)
        need = int(gr_attn.gr_decode_attn_workspace_bytes(dims))
        pl = gr_attn.plan(dims)
        refuse = False
        if need > 0:
            pairs = inp.B * Hkv
            n_qt = pl["grid"] // (8 * (-(-pairs // 8)) * pl["n_split"])
            count_bytes = pairs * n_qt * 4
            part = need - (-(-count_bytes // 256)) * 256
            refuse = count_bytes > counters or part > scratch - counters
        log(f"[noalloc random {seed}] plan={pl} workspace={need} refused={refuse}")
        out = torch.full_like(t["q"], float("nan"))
        lse = torch.full(t["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        st = gr_attn.gr_decode_attn_noalloc(
            dims, t["row_offset"].data_ptr(), t["q"].data_ptr(), t["ctx_k"].data_ptr(),
            t["ctx_v"].data_ptr(), t["ctx_len"].data_ptr(), t["beam_k"].data_ptr(),
            t["beam_v"].data_ptr(), t["beam_path"].data_ptr(), t["beam_len"].data_ptr(),
            out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if refuse:
            assert st == gr_attn.GR_ERR_WORKSPACE, (seed, gr_attn.gr_status_str(st))
            continue
        assert st == gr_attn.GR_OK, (seed, gr_attn.gr_status_str(st))
        torch.cuda.synchronize()
        ref_out, ref_lse = gr_attn.decode_attn(t["q"], t["ctx_k"], t["ctx_v"], t["ctx_len"],
                                               t["beam_k"], t["beam_v"], t["beam_path"],
                                               t["beam_len"], t["row_offset"], W_max=W_max)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), seed
        n_run += 1
    assert n_run > 0
