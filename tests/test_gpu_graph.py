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


def replays_match(call, outs, inputs_a, inputs_b, what):
    """Eager results of `call` for two input states (set by inputs_a() /
    inputs_b()), then six replays of one captured call, alternating the
    states, each checked bitwise; `outs` are the output tensors."""
    import torch
    inputs_a()
    call()
    torch.cuda.synchronize()
    ref_a = [o.clone() for o in outs]
    inputs_b()
    call()
    torch.cuda.synchronize()
    ref_b = [o.clone() for o in outs]
    assert any(not torch.equal(a, b) for a, b in zip(ref_a, ref_b)), "inputs do not matter"
    inputs_a()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    log(f"[graph] {what} captured")
    for i in range(6):
        use_b = i % 2 == 1
        (inputs_b if use_b else inputs_a)()
        for o in outs:
            o.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = ref_b if use_b else ref_a
        assert all(torch.equal(o, r) for o, r in zip(outs, ref)), f"{what}: replay {i}"
        del junk


def test_beam_select_graph_replays():
    import torch
    from shared_prefix_beam_amd import gr_attn
    si = I.select_inputs([60, 33, 90], [40, 33, 64], 3000, seed=51)
    d = "cuda"
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(d)
    ro_old, ro_new = i32(si.row_offset_old), i32(si.row_offset_new)
    score = torch.from_numpy(si.score_old).to(d)
    logits = torch.from_numpy(np.ascontiguousarray(si.logits)).to(d)
    la, lb = logits.clone(), torch.flip(logits, dims=[1]).contiguous()
    R_new, K_max = int(si.row_offset_new[-1]), 64
    outs = [torch.empty(R_new, dtype=torch.float32, device=d),
            torch.empty(R_new, dtype=torch.int32, device=d),
            torch.empty(R_new, dtype=torch.int32, device=d)]
    dims = gr_attn.SelectDims(B=3, R_old=logits.shape[0], R_new=R_new, V=logits.shape[1],
                              K_max=K_max, reserved=0)
    ws = torch.empty(gr_attn.gr_beam_select_workspace_bytes(dims), dtype=torch.uint8, device=d)

    def call():
        gr_attn.beam_select(ro_old, ro_new, score, logits, K_max, score_new=outs[0],
                            parent=outs[1], token=outs[2], workspace=ws)
    replays_match(call, outs, lambda: logits.copy_(la), lambda: logits.copy_(lb), "beam_select")


def test_beam_select_trie_graph_replays():
    import torch
    from shared_prefix_beam_amd import gr_attn
    tr = I.build_trie(I.sid_catalog(3000, 3, 300, seed=31), 300)
    ti = I.trie_select_inputs([40, 17, 60], [30, 17, 45], tr.V, 1, tr, seed=52, dead=0.1)
    si = ti.sel
    d = "cuda"
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(d)
    args = [i32(si.row_offset_old), i32(si.row_offset_new), torch.from_numpy(si.score_old).to(d)]
    logits = torch.from_numpy(np.ascontiguousarray(si.logits)).to(d)
    la, lb = logits.clone(), torch.flip(logits, dims=[1]).contiguous()
    trie = [i32(ti.node_old), i32(tr.node_ptr), i32(tr.edge_tok), i32(tr.edge_child)]
    R_new, K_max = int(si.row_offset_new[-1]), 45
    outs = [torch.empty(R_new, dtype=torch.float32, device=d)] + \
        [torch.empty(R_new, dtype=torch.int32, device=d) for _ in range(3)]
    dims = gr_attn.SelectDims(B=3, R_old=logits.shape[0], R_new=R_new, V=logits.shape[1],
                              K_max=K_max, reserved=0)
    ws = torch.empty(gr_attn.gr_beam_select_workspace_bytes(dims), dtype=torch.uint8, device=d)

    def call():
        gr_attn.beam_select_trie(*args, logits, *trie, K_max, max(tr.level_fanout(1), 1),
                                 score_new=outs[0], parent=outs[1], token=outs[2],
                                 node_new=outs[3], workspace=ws)
    replays_match(call, outs, lambda: logits.copy_(la), lambda: logits.copy_(lb),
                  "beam_select_trie")


def attention_case():
    import torch
    inp = I.custom(B=3, Hq=16, Hkv=8, D=128, W=[37, 5, 70], ctx_len=[1000, 33, 517],
                   beam_len=[3, 1, 5], seed=53)
    t = I.to_torch(inp)
    q_a, q_b = t["q"].clone(), torch.randn_like(t["q"].float()).to(torch.bfloat16)
    outs = [torch.empty_like(t["q"]),
            torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")]
    return inp, t, q_a, q_b, outs


def test_paged_graph_replays():
    import torch
    from shared_prefix_beam_amd import gr_attn
    inp, t, q_a, q_b, outs = attention_case()
    pg = I.to_paged(inp, 48, seed=54)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    kp, vp = bf(pg.k_pages), bf(pg.v_pages)
    tab = torch.from_numpy(pg.page_table.astype(np.int32)).cuda()
    W_max, tiling = int(max(inp.wl.W)), (4, 1, 3)
    dims = gr_attn.make_dims(t["q"], t["ctx_k"], t["beam_k"], t["beam_path"], W_max,
                             tiling=tiling)
    ws = torch.zeros(gr_attn.gr_decode_attn_workspace_bytes(dims), dtype=torch.uint8,
                     device="cuda")

    def call():
        gr_attn.decode_attn_paged(t["q"], kp, vp, tab, 48, t["ctx_len"], t["beam_k"],
                                  t["beam_v"], t["beam_path"], t["beam_len"], t["row_offset"],
                                  W_max=W_max, ctx_cap=inp.ctx_cap, out=outs[0], lse=outs[1],
                                  workspace=ws, tiling=tiling)
    replays_match(call, outs, lambda: t["q"].copy_(q_a), lambda: t["q"].copy_(q_b),
                  "decode_attn_paged")


def test_noalloc_graph_replays():
    import torch
    from shared_prefix_beam_amd import gr_attn
    inp, t, q_a, q_b, outs = attention_case()
    W_max = int(max(inp.wl.W))
    dims = gr_attn.make_dims(t["q"], t["ctx_k"], t["beam_k"], t["beam_path"], W_max,
                             tiling=(4, 1, 3))
    st = torch.cuda.current_stream()
    args = [gr_attn._ptr(x) for x in (t["row_offset"], t["q"], t["ctx_k"], t["ctx_v"],
                                      t["ctx_len"], t["beam_k"], t["beam_v"], t["beam_path"],
                                      t["beam_len"], outs[0], outs[1])]

    def call():
        s = torch.cuda.current_stream()
        assert gr_attn.gr_decode_attn_noalloc(dims, *args, s.cuda_stream) == gr_attn.GR_OK
    call()                                        # first call on the device: scratch set up
    torch.cuda.synchronize()
    del st
    replays_match(call, outs, lambda: t["q"].copy_(q_a), lambda: t["q"].copy_(q_b),
                  "decode_attn_noalloc")


def test_concurrent_streams():
    """Two streams (default priority) run calls at the same time, each with
    its own inputs, outputs and workspace: every result equals its eager
    call's, bitwise."""
    import torch
    from shared_prefix_beam_amd import gr_attn
    cases = []
    for k, (W, L, tiling) in enumerate(((([37, 5, 70]), [1000, 33, 517], (4, 1, 3)),
                                        (([90, 64]), [700, 1300], None))):
        inp = I.custom(B=len(W), Hq=16, Hkv=8, D=128, W=W, ctx_len=L,
                       beam_len=[3] * len(W), seed=60 + k)
        t = I.to_torch(inp)
        W_max = int(max(W))
        dims = gr_attn.make_dims(t["q"], t["ctx_k"], t["beam_k"], t["beam_path"], W_max,
                                 tiling=tiling)
        ws = torch.zeros(max(gr_attn.gr_decode_attn_workspace_bytes(dims), 256),
                         dtype=torch.uint8, device="cuda")
        cases.append((t, W_max, tiling, ws))

    def run(case, out=None, lse=None):
        t, W_max, tiling, ws = case
        return gr_attn.decode_attn(t["q"], t["ctx_k"], t["ctx_v"], t["ctx_len"], t["beam_k"],
                                   t["beam_v"], t["beam_path"], t["beam_len"], t["row_offset"],
                                   W_max=W_max, out=out, lse=lse, workspace=ws, tiling=tiling)
    refs = []
    for c in cases:
        o, l = run(c)
        torch.cuda.synchronize()
        refs.append((o.clone(), l.clone()))
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [[(torch.empty_like(r[0]), torch.empty_like(r[1])) for _ in range(8)] for r in refs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    log("[streams] two streams at once")
    for i in range(8):                           # interleaved launches on both streams
        for c, s, o in zip(cases, streams, outs):
            with torch.cuda.stream(s):
                run(c, out=o[i][0], lse=o[i][1])
    torch.cuda.synchronize()
    for r, o in zip(refs, outs):
        for i in range(8):
            assert torch.equal(o[i][0], r[0]) and torch.equal(o[i][1], r[1]), f"call {i}"
