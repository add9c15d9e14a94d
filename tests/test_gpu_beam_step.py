"""GPU parity of the beam step (BeamKV append + BeamPath update) through the
C ABI against the oracle: bit-exact (the step is integer indexing and bit
copies), including the out-of-range count."""
import numpy as np
import pytest

import pins_step
from gpu_util import assert_parity, log
from oracle import oracle as O
from shared_prefix_beam_amd import inputs as I

pytestmark = pytest.mark.gpu


def _dev(a, bf16=False):
    import torch
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a.astype(np.int32)).cuda()


def _host_bf16(t):
    return t.view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)


def gpu_step(ro_old, ro_new, parent, path_old, len_old, new_k, new_v, path_new, bk, bv, W_cap,
             count=False):
    """Run gr_beam_step on copies of the host state; return the oracle's tuple
    layout (path_new, beam_len_new, beam_k, beam_v, violations)."""
    import torch
    from shared_prefix_beam_amd import gr_attn
    B = len(ro_new) - 1
    t_path_new = _dev(path_new)
    t_len_new = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    t_bk, t_bv = _dev(bk, True), _dev(bv, True)
    viol = torch.zeros(1, dtype=torch.int32, device="cuda")
    path_old = np.asarray(path_old, dtype=np.int32).reshape(-1, np.shape(path_new)[1])
    gr_attn.beam_step(_dev(ro_old), _dev(ro_new), _dev(parent), _dev(path_old), _dev(len_old),
                      _dev(new_k, True), _dev(new_v, True), t_path_new, t_len_new, t_bk, t_bv,
                      W_cap, violations=viol)
    torch.cuda.synchronize()
    return (t_path_new.cpu().numpy(), t_len_new.cpu().numpy(), _host_bf16(t_bk),
            _host_bf16(t_bv), int(viol.item()))


def assert_same(gpu, ref, what):
    names = ("path_new", "beam_len_new", "beam_k", "beam_v", "violations")
    for n, g, r in zip(names, gpu, ref):
        if isinstance(r, int):
            assert g == r, f"{what}: {n} {g} != {r}"
        else:
            assert np.array_equal(np.asarray(g), np.asarray(r)), f"{what}: {n} differs"


def test_special_and_out_of_range_cases():
    """The oracle's special-case pin, run through the GPU: first step, a
    request with no new beams, step == T_cap, beam >= W_cap, parent == W_old."""
    log("[step] special cases")
    pins_step.pin_p4_special(gpu_step, Hkv=2, D=64)


def test_multi_step_growth_matches_oracle():
    """Five steps from empty paths with growing, shrinking and finishing
    requests: after every step the device state equals the oracle's bitwise."""
    log("[step] five-step growth")
    B, T_cap, W_cap = len(pins_step.WIDTHS), 6, 6
    dev = pins_step.grow(gpu_step, B, 8, 128, pins_step.WIDTHS, T_cap, W_cap, seed=21)
    ref = pins_step.grow(O.beam_step, B, 8, 128, pins_step.WIDTHS, T_cap, W_cap, seed=21)
    for d, r in zip(dev, ref):
        for key in ("path_new", "len_new", "bk", "bv"):
            assert np.array_equal(d[key], r[key]), (d["s"], key)
        assert d["skipped"] == r["skipped"] == 0


def test_pins_hold_on_device():
    """P1 (chain walk) and P2 (append, rest untouched) with the device step."""
    log("[step] chain walk and append pins")
    pins_step.pin_p1_chain_walk(gpu_step, Hkv=1, D=64)
    pins_step.pin_p2_append(gpu_step, Hkv=2, D=128)


@pytest.mark.parametrize("cfg", sorted(I.STEP_WORKLOADS))
def test_step_workloads_bit_exact(cfg):
    """The benchmarked step shapes (W=128 x 8 requests, W=900 x 4 requests,
    token 3), whole state compared."""
    st = I.step_workload(cfg)
    log(f"[step] workload {I.STEP_WORKLOADS[cfg]['name']} R_new={st.R_new}")
    s = st.state
    path_init = np.full((st.R_new, s.T_cap), -1, dtype=np.int32)
    args = (s.row_offset, st.row_offset_new, st.parent, s.beam_path, s.beam_len, st.new_k,
            st.new_v, path_init, s.beam_k, s.beam_v, s.W_cap)
    assert_same(gpu_step(*args), O.beam_step(*args), f"step cfg {cfg}")


def test_ragged_with_empty_requests():
    """Requests with no old beams, no new beams, first steps and later steps."""
    st = I.step_inputs(B=5, Hkv=4, D=64, W_old=[3, 0, 7, 1, 2], W_new=[5, 2, 0, 4, 1],
                       beam_len=[2, 0, 3, 4, 1], seed=77)
    log(f"[step] ragged R_new={st.R_new}")
    s = st.state
    path_init = np.full((st.R_new, s.T_cap), -1, dtype=np.int32)
    args = (s.row_offset, st.row_offset_new, st.parent, s.beam_path, s.beam_len, st.new_k,
            st.new_v, path_init, s.beam_k, s.beam_v, s.W_cap)
    assert_same(gpu_step(*args), O.beam_step(*args), "ragged")


def test_step_then_attention():
    """A state grown on the device over four steps, then decode attention on
    it, against the oracle's attention over the oracle-grown state."""
    from gpu_util import run_lib
    rng = np.random.default_rng(5)
    B, Hkv, G, D, L = 2, 8, 2, 128, 300
    widths = [[2, 5, 9, 16], [7, 7, 4, 12]]
    T_cap, W_cap = 4, 16
    log("[step] grow then attend")

    def finite(shape):
        return I.to_bf16_bits(rng.standard_normal(size=shape).astype(np.float32))

    beam_cap = T_cap * W_cap + 1
    bk0, bv0 = finite((B, beam_cap, Hkv, D)), finite((B, beam_cap, Hkv, D))
    ro = np.zeros(B + 1, dtype=np.int32)
    states = {"gpu": (np.zeros((0, T_cap), np.int32), np.zeros(B, np.int32), bk0, bv0),
              "ref": (np.zeros((0, T_cap), np.int32), np.zeros(B, np.int32), bk0, bv0)}
    for s in range(T_cap):
        w_new = [widths[b][s] for b in range(B)]
        ro_new = np.zeros(B + 1, dtype=np.int32)
        ro_new[1:] = np.cumsum(w_new)
        parent = np.concatenate([rng.integers(0, max(int(ro[b + 1] - ro[b]), 1), size=w_new[b])
                                 for b in range(B)]).astype(np.int32)
        nk, nv = finite((int(ro_new[-1]), Hkv, D)), finite((int(ro_new[-1]), Hkv, D))
        init = np.full((int(ro_new[-1]), T_cap), -1, np.int32)
        for key, fn in (("gpu", gpu_step), ("ref", O.beam_step)):
            path, ln, bk, bv = states[key]
            p2, l2, bk2, bv2, sk = fn(ro, ro_new, parent, path, ln, nk, nv, init, bk, bv, W_cap)
            assert sk == 0
            states[key] = (p2, l2, bk2, bv2)
        ro = ro_new
    for a, b in zip(states["gpu"], states["ref"]):
        assert np.array_equal(a, b)
    path, ln, bk, bv = states["gpu"]
    R = int(ro[-1])
    inp = I.custom(B=B, Hq=Hkv * G, Hkv=Hkv, D=D, W=[widths[b][-1] for b in range(B)],
                   ctx_len=[L, L - 77], beam_len=[T_cap] * B, seed=6, T_cap=T_cap, W_cap=W_cap)
    inp.beam_k, inp.beam_v, inp.beam_path, inp.beam_len = bk, bv, path, ln
    out, lse = run_lib(inp, "fused")
    ref_out, ref_lse = O.decode_attn_inputs(inp)
    assert out.shape == (R, Hkv * G, D)
    assert_parity(out, lse, ref_out, ref_lse, "grown state")
