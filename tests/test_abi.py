"""The C-ABI library on the CPU: it loads, exports every declared symbol and
rejects bad arguments in host validation, before touching the GPU."""
import ctypes
import os
import re

import pytest

from shared_prefix_beam_amd import gr_attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gr_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gr_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return gr_attn.load()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(gr_attn.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_dims_struct_layout():
    # int32 x8, int64 x2, float, int32, pointer, uint64 -> 72 bytes, 8-aligned
    assert ctypes.sizeof(gr_attn.Dims) == 72
    assert gr_attn.Dims.ctx_cap.offset == 32 and gr_attn.Dims.scale.offset == 48
    assert gr_attn.Dims.workspace.offset == 56 and gr_attn.Dims.workspace_bytes.offset == 64


def test_version_and_status_strings(lib):
    assert gr_attn.gr_version() >= 100
    assert gr_attn.gr_status_str(0) == "ok"
    for code in (-1, -2, -3, -4, -5, -6, -7):
        assert gr_attn.gr_status_str(code) != "unknown status"


def good_dims(**over):
    d = dict(B=2, R=10, Hq=16, Hkv=8, D=128, W_max=5, T_cap=3, reserved=0, ctx_cap=64,
             beam_cap=16, scale=0.0, flags=0)
    d.update(over)
    return gr_attn.Dims(**d)


P16 = 0x10000        # fake, aligned, never dereferenced: validation fails first


def call(dims, **ptrs):
    args = dict(row_offset=P16, q=P16, ctx_k=P16, ctx_v=P16, ctx_len=P16, beam_k=P16,
                beam_v=P16, beam_path=P16, beam_len=P16, out=P16, lse=P16)
    args.update(ptrs)
    return gr_attn.gr_decode_attn(dims, args["row_offset"], args["q"], args["ctx_k"],
                                  args["ctx_v"], args["ctx_len"], args["beam_k"],
                                  args["beam_v"], args["beam_path"], args["beam_len"],
                                  args["out"], args["lse"], None)


@pytest.mark.parametrize("over,code", [
    (dict(Hq=12, Hkv=8), gr_attn.GR_ERR_DIMS),
    (dict(R=-1), gr_attn.GR_ERR_DIMS),
    (dict(B=-1), gr_attn.GR_ERR_DIMS),
    (dict(scale=-1.0), gr_attn.GR_ERR_DIMS),
    (dict(scale=float("nan")), gr_attn.GR_ERR_DIMS),
    (dict(reserved=1), gr_attn.GR_ERR_DIMS),
    (dict(flags=2), gr_attn.GR_ERR_DIMS),
    (dict(flags=gr_attn.tiling_flags((4, 1, 9))), gr_attn.GR_ERR_DIMS),
    (dict(flags=gr_attn.tiling_flags((0, 1, 1))), gr_attn.GR_ERR_DIMS),
    (dict(flags=gr_attn.tiling_flags((4, 1, 1)) | (1 << 24)), gr_attn.GR_ERR_DIMS),
    (dict(flags=gr_attn.tiling_flags((3, 3, 1))), gr_attn.GR_ERR_UNSUPPORTED),
    (dict(flags=gr_attn.tiling_flags((2, 4, 1))), gr_attn.GR_ERR_UNSUPPORTED),
    (dict(D=96), gr_attn.GR_ERR_UNSUPPORTED),
    (dict(Hq=32, Hkv=2), gr_attn.GR_ERR_UNSUPPORTED),
])
def test_bad_dims_rejected(over, code):
    assert call(good_dims(**over)) == code


def test_null_and_alignment_rejected():
    assert gr_attn.load().gr_decode_attn(None, *([P16] * 11), None) == gr_attn.GR_ERR_NULL
    assert call(good_dims(), q=None) == gr_attn.GR_ERR_NULL
    assert call(good_dims(), row_offset=None) == gr_attn.GR_ERR_NULL
    assert call(good_dims(), ctx_k=P16 + 8) == gr_attn.GR_ERR_ALIGN
    assert call(good_dims(), out=P16 + 2) == gr_attn.GR_ERR_ALIGN
    assert call(good_dims(), lse=P16 + 2) == gr_attn.GR_ERR_ALIGN


def split_dims(**over):
    # 16 (request, KV head) pairs of 10 stacked rows and 8192 context tokens:
    # far too few waves for the GPU, and partials much smaller than the
    # context, so each pair's context is split
    d = dict(B=2, R=10, Hq=16, Hkv=8, D=128, W_max=5, T_cap=3, reserved=0, ctx_cap=8192,
             beam_cap=16, scale=0.0, flags=0)
    d.update(over)
    return gr_attn.Dims(**d)


def part_bytes(D):
    return (D // 8 + 1) * 64 * 16       # one wave's partial: O^T fragments + stats


def test_workspace_bytes():
    f = gr_attn.gr_decode_attn_workspace_bytes
    assert f(good_dims()) == 0                               # 2 context tiles: no split
    assert f(split_dims()) > 0
    assert f(good_dims(R=0, W_max=0)) == 0 and f(split_dims(Hq=12)) == 0
    assert gr_attn.load().gr_decode_attn_workspace_bytes(None) == 0
    # forced tilings: counters (256-byte aligned) + units x splits x waves partials
    for nqt, nks, sp in ((4, 1, 1), (4, 1, 3), (2, 2, 8), (8, 1, 2)):
        n = f(split_dims(flags=gr_attn.tiling_flags((nqt, nks, sp))))
        units = 2 * 8 * -(-10 // (32 * nqt))
        want = 0 if sp == 1 else ((units * 4 + 255) // 256) * 256 + units * sp * nqt * \
            part_bytes(128)
        assert n == want, (nqt, nks, sp, n, want)


def workload_dims(cfg):
    from shared_prefix_beam_amd import inputs as I
    wl = I.WORKLOADS[cfg]
    return gr_attn.Dims(B=wl.B, R=sum(wl.W), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, W_max=max(wl.W),
                        T_cap=wl.T[-1], reserved=0, ctx_cap=wl.ctx[-1], beam_cap=16,
                        scale=0.0, flags=0)


# (nqt, nks, n_split, row16) the planner takes for the five workloads: waves
# of 16 rows with two key streams where no 32-row tiling fills two waves per
# SIMD (1 request of 4 beams, 8 requests of 128), else (4,1) of 32-row waves
@pytest.mark.parametrize("cfg,want", [(1, (4, 2, 1, 1)), (2, (4, 2, 1, 1)), (3, (4, 1, 1, 0)),
                                      (4, (4, 1, 1, 0)), (5, (4, 1, 1, 0))])
def test_planner_choices(cfg, want):
    p = gr_attn.plan(workload_dims(cfg))
    assert (p["nqt"], p["nks"], p["n_split"], int(p["row16"])) == want
    d = workload_dims(cfg)
    pairs = d.B * d.Hkv
    rows = (16 if p["row16"] else 32) * p["nqt"]
    n_qt = -(-(d.W_max * (d.Hq // d.Hkv)) // rows)
    assert p["grid"] == 8 * -(-pairs // 8) * n_qt * p["n_split"]


def test_plan_echoes_forced_tilings_and_rejects_bad_ones(lib):
    p = gr_attn.plan(good_dims(flags=gr_attn.tiling_flags((4, 2, 1, True))))
    assert (p["nqt"], p["nks"], p["n_split"], p["row16"]) == (4, 2, 1, True)
    p = gr_attn.plan(split_dims(flags=gr_attn.tiling_flags((4, 1, 4))))
    assert (p["nqt"], p["nks"], p["n_split"], p["row16"]) == (4, 1, 4, False)
    p = gr_attn.plan(split_dims())
    assert p["n_split"] > 1                      # few pairs, long context: split
    assert gr_attn.plan(good_dims(R=0, W_max=0))["grid"] == 0
    out = (ctypes.c_int32 * 5)()
    assert lib.gr_decode_attn_plan(ctypes.byref(good_dims()), None) == gr_attn.GR_ERR_NULL
    assert lib.gr_decode_attn_plan(None, out) == gr_attn.GR_ERR_NULL
    assert lib.gr_decode_attn_plan(ctypes.byref(good_dims(Hq=12)), out) == gr_attn.GR_ERR_DIMS
    st = lib.gr_decode_attn_plan(ctypes.byref(good_dims(flags=gr_attn.tiling_flags((3, 3, 1)))),
                                 out)
    assert st == gr_attn.GR_ERR_UNSUPPORTED


def test_workspace_rejected():
    need = gr_attn.gr_decode_attn_workspace_bytes(split_dims())
    assert call(split_dims()) == gr_attn.GR_ERR_WORKSPACE                     # NULL
    assert call(split_dims(workspace=P16 * 16, workspace_bytes=need - 1)) == \
        gr_attn.GR_ERR_WORKSPACE                                              # short
    assert call(split_dims(workspace=P16 * 16 + 128, workspace_bytes=need)) == \
        gr_attn.GR_ERR_WORKSPACE                                              # misaligned
    # accepted: validation passes and only the (absent) device is refused
    assert call(split_dims(workspace=P16 * 16, workspace_bytes=need)) in (
        gr_attn.GR_ERR_DEVICE, gr_attn.GR_ERR_UNSUPPORTED)


def test_empty_call_is_a_no_op():
    # nothing to compute: returns before any device access
    assert call(good_dims(R=0, W_max=0)) == gr_attn.GR_OK


def test_generic_rejects_too_long_context():
    d = good_dims(ctx_cap=20000)
    st = gr_attn.gr_decode_attn_generic(d, *([P16] * 11), None)
    assert st == gr_attn.GR_ERR_UNSUPPORTED


# ---- gr_beam_step host validation ------------------------------------------
def test_step_dims_struct_layout():
    # int32 x8, int64 -> 40 bytes, beam_cap at 32
    assert ctypes.sizeof(gr_attn.StepDims) == 40
    assert gr_attn.StepDims.beam_cap.offset == 32


def step_dims(**over):
    d = dict(B=2, R_old=6, R_new=8, Hkv=8, D=128, T_cap=4, W_cap=4, reserved=0, beam_cap=17)
    d.update(over)
    return gr_attn.StepDims(**d)


def step_call(dims, **ptrs):
    # path_old and path_new in separate fake ranges (R * T_cap * 4 bytes apart)
    args = dict(ro_old=P16, ro_new=P16, parent=P16, path_old=P16, len_old=P16, new_k=P16,
                new_v=P16, path_new=P16 * 2, len_new=P16 * 3, beam_k=P16, beam_v=P16,
                violations=None)
    args.update(ptrs)
    return gr_attn.gr_beam_step(dims, args["ro_old"], args["ro_new"], args["parent"],
                                args["path_old"], args["len_old"], args["new_k"], args["new_v"],
                                args["path_new"], args["len_new"], args["beam_k"],
                                args["beam_v"], args["violations"], None)


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), gr_attn.GR_ERR_DIMS),
    (dict(R_new=-1), gr_attn.GR_ERR_DIMS),
    (dict(Hkv=0), gr_attn.GR_ERR_DIMS),
    (dict(W_cap=-1), gr_attn.GR_ERR_DIMS),
    (dict(beam_cap=-1), gr_attn.GR_ERR_DIMS),
    (dict(reserved=3), gr_attn.GR_ERR_DIMS),
    (dict(D=96), gr_attn.GR_ERR_UNSUPPORTED),
])
def test_step_bad_dims_rejected(over, code):
    assert step_call(step_dims(**over)) == code


@pytest.mark.parametrize("which", ["ro_old", "ro_new", "parent", "new_k", "new_v", "path_new",
                                   "len_old", "len_new", "beam_k", "beam_v", "path_old"])
def test_step_null_pointer_rejected(which):
    assert step_call(step_dims(), **{which: None}) == gr_attn.GR_ERR_NULL


def test_step_null_dims_rejected():
    assert gr_attn.load().gr_beam_step(None, *([None] * 13)) == gr_attn.GR_ERR_NULL


@pytest.mark.parametrize("which", ["new_k", "beam_v"])
def test_step_misaligned_bf16_rejected(which):
    assert step_call(step_dims(), **{which: P16 + 8}) == gr_attn.GR_ERR_ALIGN


def test_step_overlapping_tables_rejected():
    # path_new starting inside path_old's R_old * T_cap * 4 bytes
    assert step_call(step_dims(), path_new=P16 + 16) == gr_attn.GR_ERR_DIMS
    assert step_call(step_dims(), len_new=P16 + 4, len_old=P16) == gr_attn.GR_ERR_DIMS


def test_step_empty_batch_is_a_no_op():
    assert step_call(step_dims(B=0, R_old=0, R_new=0)) == gr_attn.GR_OK


# ---- gr_decode_attn_paged host validation ----------------------------------
def paged_call(dims, ctx):
    return gr_attn.gr_decode_attn_paged(dims, ctx, P16, P16, P16, P16, P16, P16, P16, P16, P16,
                                        None)


def good_ctx(**over):
    c = dict(k_pages=P16, v_pages=P16, page_table=P16, page_size=16, pages_per_req=4,
             n_pages=9)
    c.update(over)
    return gr_attn.PagedCtx(**c)


def test_paged_ctx_struct_layout():
    assert ctypes.sizeof(gr_attn.PagedCtx) == 40
    assert gr_attn.PagedCtx.n_pages.offset == 32


@pytest.mark.parametrize("over,code", [
    (dict(page_size=24), gr_attn.GR_ERR_DIMS),
    (dict(page_size=0), gr_attn.GR_ERR_DIMS),
    (dict(pages_per_req=0), gr_attn.GR_ERR_DIMS),
    (dict(n_pages=0), gr_attn.GR_ERR_DIMS),
    (dict(pages_per_req=3), gr_attn.GR_ERR_DIMS),     # ctx_cap 64 > 3 * 16
    (dict(k_pages=None), gr_attn.GR_ERR_NULL),
    (dict(page_table=None), gr_attn.GR_ERR_NULL),
    (dict(v_pages=P16 + 8), gr_attn.GR_ERR_ALIGN),
])
def test_paged_bad_ctx_rejected(over, code):
    assert paged_call(good_dims(), good_ctx(**over)) == code


def test_paged_null_ctx_rejected():
    assert gr_attn.load().gr_decode_attn_paged(ctypes.byref(good_dims()), None,
                                               *([None] * 10)) == gr_attn.GR_ERR_NULL


# ---- gr_beam_select host validation ----------------------------------------
def test_select_dims_struct_layout():
    assert ctypes.sizeof(gr_attn.SelectDims) == 24


def select_dims(**over):
    d = dict(B=2, R_old=6, R_new=8, V=1000, K_max=5, reserved=0)
    d.update(over)
    return gr_attn.SelectDims(**d)


def select_call(dims, ws_bytes=None, **ptrs):
    args = dict(ro_old=P16, ro_new=P16, score_old=P16, logits=P16, score_new=P16, parent=P16,
                token=P16, workspace=P16)
    args.update(ptrs)
    if ws_bytes is None:
        ws_bytes = gr_attn.gr_beam_select_workspace_bytes(dims)
    return gr_attn.gr_beam_select(dims, args["ro_old"], args["ro_new"], args["score_old"],
                                  args["logits"], args["score_new"], args["parent"],
                                  args["token"], args["workspace"], ws_bytes, None)


def test_select_workspace_size():
    # per row: a 32-key list (8 bytes each), its fp32 offset, an int32 slot,
    # K_max survivor keys, its candidate count and first trie edge; six
    # tables, each rounded up to 256 bytes
    def al(n):
        return (n + 255) // 256 * 256

    for R, K in ((6, 5), (900, 900), (1, 1024)):
        want = al(R * 32 * 8) + al(R * 4) + al(R * 4) + al(R * K * 8) + 2 * al(R * 4)
        assert gr_attn.gr_beam_select_workspace_bytes(select_dims(R_old=R, K_max=K)) == want
    assert gr_attn.gr_beam_select_workspace_bytes(select_dims(R_old=900, K_max=900)) == \
        6718208 + 2 * 3840
    assert gr_attn.gr_beam_select_workspace_bytes(select_dims(R_old=0)) == 0
    assert gr_attn.load().gr_beam_select_workspace_bytes(None) == 0


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), gr_attn.GR_ERR_DIMS),
    (dict(R_old=-1), gr_attn.GR_ERR_DIMS),
    (dict(R_new=-1), gr_attn.GR_ERR_DIMS),
    (dict(V=0), gr_attn.GR_ERR_DIMS),
    (dict(K_max=0), gr_attn.GR_ERR_DIMS),
    (dict(reserved=1), gr_attn.GR_ERR_DIMS),
    (dict(V=16385), gr_attn.GR_ERR_UNSUPPORTED),
    (dict(K_max=1025), gr_attn.GR_ERR_UNSUPPORTED),
    (dict(R_old=200000, V=16384), gr_attn.GR_ERR_UNSUPPORTED),
])
def test_select_bad_dims_rejected(over, code):
    assert select_call(select_dims(**over), ws_bytes=1 << 40) == code


@pytest.mark.parametrize("which", ["ro_old", "ro_new", "score_old", "logits", "score_new",
                                   "parent", "token", "workspace"])
def test_select_null_pointer_rejected(which):
    assert select_call(select_dims(), **{which: None}) == gr_attn.GR_ERR_NULL


def test_select_null_dims_rejected():
    assert gr_attn.load().gr_beam_select(None, *([None] * 8), 0, None) == gr_attn.GR_ERR_NULL


def test_select_short_workspace_rejected():
    d = select_dims()
    assert select_call(d, ws_bytes=gr_attn.gr_beam_select_workspace_bytes(d) - 1) == \
        gr_attn.GR_ERR_DIMS


@pytest.mark.parametrize("which,off", [("logits", 2), ("token", 1), ("workspace", 8)])
def test_select_misaligned_rejected(which, off):
    assert select_call(select_dims(), **{which: P16 + off}) == gr_attn.GR_ERR_ALIGN


def test_select_empty_batch_is_a_no_op():
    assert select_call(select_dims(B=0, R_old=0, R_new=0)) == gr_attn.GR_OK


# ---- gr_beam_select_trie host validation -----------------------------------
def test_trie_struct_layout():
    assert ctypes.sizeof(gr_attn.SidTrie) == 40


def trie_desc(**over):
    d = dict(node_ptr=P16, edge_tok=P16, edge_child=P16, n_nodes=10, n_edges=9, max_fanout=4,
             reserved=0)
    d.update(over)
    return gr_attn.SidTrie(**d)


def trie_call(dims, trie, **ptrs):
    args = dict(ro_old=P16, ro_new=P16, score_old=P16, logits=P16, node_old=P16,
                score_new=P16, parent=P16, token=P16, node_new=P16, workspace=P16)
    args.update(ptrs)
    return gr_attn.gr_beam_select_trie(dims, trie, args["ro_old"], args["ro_new"],
                                       args["score_old"], args["logits"], args["node_old"],
                                       args["score_new"], args["parent"], args["token"],
                                       args["node_new"], args["workspace"],
                                       gr_attn.gr_beam_select_workspace_bytes(dims), None)


@pytest.mark.parametrize("over,code", [
    (dict(n_nodes=0), gr_attn.GR_ERR_DIMS),
    (dict(n_edges=-1), gr_attn.GR_ERR_DIMS),
    (dict(max_fanout=0), gr_attn.GR_ERR_DIMS),
    (dict(max_fanout=1001), gr_attn.GR_ERR_DIMS),
    (dict(reserved=2), gr_attn.GR_ERR_DIMS),
    (dict(node_ptr=None), gr_attn.GR_ERR_NULL),
    (dict(edge_tok=None), gr_attn.GR_ERR_NULL),
    (dict(edge_child=P16 + 2), gr_attn.GR_ERR_ALIGN),
])
def test_trie_bad_descriptor_rejected(over, code):
    assert trie_call(select_dims(), trie_desc(**over)) == code


@pytest.mark.parametrize("which", ["node_old", "node_new", "logits", "workspace"])
def test_trie_null_pointer_rejected(which):
    assert trie_call(select_dims(), trie_desc(), **{which: None}) == gr_attn.GR_ERR_NULL


def test_trie_null_descriptor_rejected():
    lib = gr_attn.load()
    assert lib.gr_beam_select_trie(ctypes.byref(select_dims()), None, *([None] * 10), 0,
                                   None) == gr_attn.GR_ERR_NULL


def test_trie_empty_batch_is_a_no_op():
    assert trie_call(select_dims(B=0, R_old=0, R_new=0), trie_desc()) == gr_attn.GR_OK


def test_noalloc_rejects_split_beyond_scratch():
    # 64 requests x 8 KV heads x 15 query tiles forced into 8 splits: partials
    # of ~1 GB cannot fit the 16 MiB scratch; refused before any device access
    d = good_dims(B=64, R=64 * 900, W_max=900, ctx_cap=2048, flags=gr_attn.tiling_flags((4, 1, 8)))
    st = gr_attn.gr_decode_attn_noalloc(d, *([P16] * 11), None)
    assert st == gr_attn.GR_ERR_WORKSPACE
    # without a split there is nothing to place: validation passes, the
    # missing device is what is refused
    d = good_dims(flags=gr_attn.tiling_flags((4, 1, 1)))
    assert gr_attn.gr_decode_attn_noalloc(d, *([P16] * 11), None) in (
        gr_attn.GR_ERR_DEVICE, gr_attn.GR_ERR_UNSUPPORTED)
