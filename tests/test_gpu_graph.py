"""The entry points are capturable into a HIP graph (they enqueue work only:
no allocation, synchronisation or host reads).  A captured call is replayed
several times, with other eager work and synchronisations between the
replays, and every replay must reproduce the eager result bitwise; the
inputs change between replays to show that the graph reads them anew."""
import numpy as np
import pytest

from gpu_util import log
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_decode_attn_graph_replays():
    import torch
    from shared_prefix_beam_amd import gr_attn
    inp = I.custom(B=3, Hq=16, Hkv=8, D=128, W=[37, 5, 70], ctx_len=[1000, 33, 517],
                   beam_len=[3, 1, 5], seed=41)
    t = I.to_torch(inp)
    W_max = int(max(inp.wl.W))
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    q_other = torch.randn_like(t["q"].float()).to(torch.bfloat16)
    q_orig = t["q"].clone()
    # each pair's context split over 4 workgroups: one workspace, zeroed
    # once, serves every call and replay (its counters reset themselves)
    tiling = (4, 1, 4)
    dims = gr_attn.make_dims(t["q"], t["ctx_k"], t["beam_k"], t["beam_path"], W_max,
                             tiling=tiling)
    need = gr_attn.gr_decode_attn_workspace_bytes(dims)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")

    def call():
        gr_attn.decode_attn(t["q"], t["ctx_k"], t["ctx_v"], t["ctx_len"], t["beam_k"],
                            t["beam_v"], t["beam_path"], t["beam_len"], t["row_offset"],
                            W_max=W_max, out=out, lse=lse, workspace=ws, tiling=tiling)

    # eager references for both query sets
    call()
    torch.cuda.synchronize()
    ref_a = (out.clone(), lse.clone())
    t["q"].copy_(q_other)
    call()
    torch.cuda.synchronize()
    ref_b = (out.clone(), lse.clone())
    t["q"].copy_(q_orig)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    log("[graph] decode_attn captured")
    for i in range(6):
        use_b = i % 2 == 1
        t["q"].copy_(q_other if use_b else q_orig)
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = ref_b if use_b else ref_a
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {i}"
        del junk
    # every arrival counter is back at zero
    n_counters = 3 * 8 * 2                       # pairs x query tiles of the (4,1) plan
    assert int(ws[:4 * n_counters].view(torch.int32).abs().sum()) == 0


def test_beam_step_graph_replays():
    import torch
    from shared_prefix_beam_amd import gr_attn
    st = I.step_inputs(B=3, Hkv=8, D=128, W_old=[9, 4, 12], W_new=[12, 3, 7],
                       beam_len=[2, 1, 3], seed=42)
    s_ = st.state

    def dev(a, bf=False):
        a = np.ascontiguousarray(a)
        if bf:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a.astype(np.int32)).cuda()

    args = dict(ro_old=dev(s_.row_offset), ro_new=dev(st.row_offset_new), parent=dev(st.parent),
                path_old=dev(s_.beam_path), len_old=dev(s_.beam_len), new_k=dev(st.new_k, True),
                new_v=dev(st.new_v, True))
    path_new = torch.full((st.R_new, s_.T_cap), -1, dtype=torch.int32, device="cuda")
    len_new = torch.zeros(s_.B, dtype=torch.int32, device="cuda")
    bk0, bv0 = dev(s_.beam_k, True), dev(s_.beam_v, True)
    bk, bv = bk0.clone(), bv0.clone()

    def call():
        gr_attn.beam_step(args["ro_old"], args["ro_new"], args["parent"], args["path_old"],
                          args["len_old"], args["new_k"], args["new_v"], path_new, len_new, bk, bv,
                          s_.W_cap)

    call()
    torch.cuda.synchronize()
    ref = (path_new.clone(), len_new.clone(), bk.clone(), bv.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    log("[graph] beam_step captured")
    for i in range(5):
        path_new.fill_(-1)
        len_new.zero_()
        bk.copy_(bk0)
        bv.copy_(bv0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((path_new, len_new, bk, bv), ref):
            if a.dtype == torch.bfloat16:           # NaN padding: compare the bits
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"replay {i}"


def test_non_default_stream():
    import torch
    from gpu_util import run_lib
    from shared_prefix_beam_amd import gr_attn
    inp = I.custom(B=2, Hq=16, Hkv=8, D=128, W=[20, 9], ctx_len=[300, 77], beam_len=[2, 3],
                   seed=43)
    ref_out, ref_lse = run_lib(inp, "fused")
    t = I.to_torch(inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out, lse = gr_attn.decode_attn(t["q"], t["ctx_k"], t["ctx_v"], t["ctx_len"], t["beam_k"],
                                       t["beam_v"], t["beam_path"], t["beam_len"],
                                       t["row_offset"], W_max=20)
    s.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), ref_out)
    assert np.array_equal(lse.cpu().numpy(), ref_lse)
