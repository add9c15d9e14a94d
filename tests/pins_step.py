"""Independent checks that pin the beam-step oracle (BeamKV append + BeamPath
update); not a test module itself.

Each ``pin_*`` takes a callable with the signature of ``oracle.beam_step``
and raises ``AssertionError`` on a disagreement with something fixed
independently of the oracle's own indexing:

* P1  chain walk: a state grown step by step from empty paths, with the
      recorded parent choices, gives every row the path found by walking its
      parents back to step 0 (slot of step s, beam k = s*W_cap + k)
* P2  append: each new row's K/V land bitwise in its step slot; every other
      BeamKV element keeps its bits
* P3  composition: attention over the grown state equals plain softmax
      attention (torch SDPA, fp64) over context ++ the K/V each beam drew at
      every step of its ancestry
* P4  special cases: first step, a request with no new beams, path entries
      past the new length untouched, out-of-range rows skipped and counted
"""
from __future__ import annotations

from typing import Callable, List

import numpy as np
import torch

from shared_prefix_beam_amd import inputs as I

StepFn = Callable[..., tuple]


def _apply(fn: StepFn, ro_old, ro_new, parent, path_old, len_old, new_k, new_v, path_new, bk, bv,
           W_cap):
    return fn(ro_old, ro_new, parent, path_old, len_old, new_k, new_v, path_new, bk, bv, W_cap)


def grow(fn: StepFn, B: int, Hkv: int, D: int, widths: List[List[int]], T_cap: int, W_cap: int,
         seed: int):
    """Run len(widths[0]) steps from empty paths.  widths[b][s] = beams of
    request b at step s.  Returns per-step records for the pins."""
    rng = np.random.default_rng(seed)
    n_steps = len(widths[0])
    beam_cap = T_cap * W_cap + 1
    bk = rng.integers(0, 1 << 16, size=(B, beam_cap, Hkv, D), dtype=np.uint16)
    bv = rng.integers(0, 1 << 16, size=(B, beam_cap, Hkv, D), dtype=np.uint16)
    ro = np.zeros(B + 1, dtype=np.int32)
    path = np.zeros((0, T_cap), dtype=np.int32)
    length = np.zeros(B, dtype=np.int32)
    steps = []
    for s in range(n_steps):
        w_new = np.array([widths[b][s] for b in range(B)], dtype=np.int64)
        ro_new = np.zeros(B + 1, dtype=np.int32)
        ro_new[1:] = np.cumsum(w_new)
        R_new = int(ro_new[-1])
        parent = np.zeros(R_new, dtype=np.int32)
        for b in range(B):
            w_old = int(ro[b + 1] - ro[b])
            if w_new[b] and s > 0 and w_old > 0:
                parent[ro_new[b]:ro_new[b + 1]] = rng.integers(0, w_old, size=int(w_new[b]))
        new_k = rng.integers(0, 1 << 16, size=(R_new, Hkv, D), dtype=np.uint16)
        new_v = rng.integers(0, 1 << 16, size=(R_new, Hkv, D), dtype=np.uint16)
        path_init = rng.integers(-5, 5, size=(R_new, T_cap), dtype=np.int32)
        path_new, len_new, bk2, bv2, skipped = _apply(fn, ro, ro_new, parent, path, length, new_k,
                                                      new_v, path_init, bk, bv, W_cap)
        steps.append(dict(s=s, ro_old=ro, ro_new=ro_new, parent=parent, new_k=new_k,
                          new_v=new_v, path_init=path_init, path_new=path_new, len_old=length,
                          len_new=len_new, bk_old=bk, bv_old=bv, bk=bk2, bv=bv2,
                          skipped=skipped))
        ro, path, length, bk, bv = ro_new, path_new, len_new, bk2, bv2
    return steps


# request 0 keeps 3 beams, request 1 grows 1 -> 6, request 2 stops after two
# steps, request 3 shrinks 5 -> 2
WIDTHS = [[3, 3, 3, 3, 3], [1, 2, 4, 5, 6], [4, 4, 0, 0, 0], [5, 4, 3, 2, 2]]


def pin_p1_chain_walk(fn: StepFn, seed: int = 3, Hkv: int = 2, D: int = 8):
    B, T_cap, W_cap = len(WIDTHS), 6, 6
    steps = grow(fn, B, Hkv, D, WIDTHS, T_cap, W_cap, seed)
    for st in steps:
        s = st["s"]
        assert st["skipped"] == 0
        for b in range(B):
            assert st["len_new"][b] == (s + 1 if WIDTHS[b][s] > 0 else st["len_old"][b])
            for k in range(WIDTHS[b][s]):
                # walk back through the recorded parent choices
                slots, kk = [], k
                for ss in range(s, -1, -1):
                    slots.append(ss * W_cap + kk)
                    if ss > 0:
                        par = steps[ss]["parent"]
                        kk = int(par[steps[ss]["ro_new"][b] + kk])
                slots.reverse()
                r = int(st["ro_new"][b]) + k
                assert list(st["path_new"][r, :s + 1]) == slots, (s, b, k)
                # entries past the new length keep what the table held
                assert np.array_equal(st["path_new"][r, s + 1:], st["path_init"][r, s + 1:])


def pin_p2_append(fn: StepFn, seed: int = 4, Hkv: int = 3, D: int = 16):
    B, T_cap, W_cap = len(WIDTHS), 6, 6
    steps = grow(fn, B, Hkv, D, WIDTHS, T_cap, W_cap, seed)
    for st in steps:
        s = st["s"]
        written = np.zeros(st["bk"].shape[:2], dtype=bool)
        for b in range(B):
            for k in range(WIDTHS[b][s]):
                r = int(st["ro_new"][b]) + k
                slot = s * W_cap + k
                assert np.array_equal(st["bk"][b, slot], st["new_k"][r])
                assert np.array_equal(st["bv"][b, slot], st["new_v"][r])
                written[b, slot] = True
        assert np.array_equal(st["bk"][~written], st["bk_old"][~written])
        assert np.array_equal(st["bv"][~written], st["bv_old"][~written])


def _sdpa(q, K, V, scale):
    qt = torch.from_numpy(q)[None, None, None, :]
    Kt = torch.from_numpy(K)[None, None]
    Vt = torch.from_numpy(V)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return o[0, 0, 0].numpy()


def pin_p3_composition(fn: StepFn, seed: int = 5):
    from oracle import oracle as O
    B, Hkv, D, G = 2, 2, 8, 2
    widths = [[2, 3, 3, 4], [3, 3, 2, 2]]
    T_cap, W_cap = 4, 4
    # finite values only (the random-bit caches of ``grow`` may hold NaN)
    rng = np.random.default_rng(seed)
    steps = grow(fn, B, Hkv, D, widths, T_cap, W_cap, seed)
    fin = lambda a: I.to_bf16_bits(rng.standard_normal(size=a.shape).astype(np.float32))
    # redo the growth with finite K/V: replay the recorded parents
    bk = fin(steps[0]["bk_old"])
    bv = fin(steps[0]["bv_old"])
    ro = np.zeros(B + 1, dtype=np.int32)
    path = np.zeros((0, T_cap), dtype=np.int32)
    length = np.zeros(B, dtype=np.int32)
    drawn = []
    for st in steps:
        nk, nv = fin(st["new_k"]), fin(st["new_v"])
        drawn.append((nk, nv))
        path, length, bk, bv, sk = _apply(fn, ro, st["ro_new"], st["parent"], path, length, nk,
                                          nv, st["path_init"], bk, bv, W_cap)
        assert sk == 0
        ro = st["ro_new"]
    L = 5
    ctx_k = fin(np.zeros((B, L, Hkv, D), dtype=np.uint16))
    ctx_v = fin(np.zeros((B, L, Hkv, D), dtype=np.uint16))
    R = int(ro[-1])
    q = fin(np.zeros((R, Hkv * G, D), dtype=np.uint16))
    out, lse = O.decode_attn(q, ctx_k, ctx_v, np.full(B, L, np.int32), bk, bv, path, length, ro)
    f = lambda a: I.bf16_bits_to_f32(a).astype(np.float64)
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        for k in range(widths[b][-1]):
            r = int(ro[b]) + k
            # the K/V this beam drew at each step of its ancestry
            chain, kk = [], k
            for si in range(len(steps) - 1, -1, -1):
                chain.append((si, int(steps[si]["ro_new"][b]) + kk))
                if si > 0:
                    kk = int(steps[si]["parent"][steps[si]["ro_new"][b] + kk])
            chain.reverse()
            for h in range(Hkv * G):
                g = h // G
                K = np.concatenate([f(ctx_k[b, :, g])] + [f(drawn[si][0][rr, g])[None] for si, rr in chain])
                V = np.concatenate([f(ctx_v[b, :, g])] + [f(drawn[si][1][rr, g])[None] for si, rr in chain])
                ref = _sdpa(f(q[r, h]), K, V, scale)
                assert np.max(np.abs(out[r, h] - ref)) < 1e-12, (b, k, h)


def pin_p4_special(fn: StepFn, Hkv: int = 1, D: int = 4):
    rng = np.random.default_rng(9)
    B, T_cap, W_cap = 3, 3, 4
    beam_cap = T_cap * W_cap + 1
    bk = rng.integers(0, 1 << 16, size=(B, beam_cap, Hkv, D), dtype=np.uint16)
    bv = bk.copy()
    # first step for request 0 (no old rows), request 1 with no new beams,
    # request 2 at step 1
    ro_old = np.array([0, 0, 2, 4], dtype=np.int32)
    path_old = np.array([[0, 9, 9], [1, 9, 9], [2, 9, 9], [3, 9, 9]], dtype=np.int32)
    len_old = np.array([0, 1, 1], dtype=np.int32)
    ro_new = np.array([0, 2, 2, 5], dtype=np.int32)
    parent = np.array([7, 7, 1, 0, 1], dtype=np.int32)
    new_k = rng.integers(0, 1 << 16, size=(5, Hkv, D), dtype=np.uint16)
    path_init = np.full((5, T_cap), -3, dtype=np.int32)
    p, ln, bk2, bv2, sk = fn(ro_old, ro_new, parent, path_old, len_old, new_k, new_k, path_init,
                             bk, bv, W_cap)
    assert sk == 0
    assert list(ln) == [1, 1, 2]
    assert list(p[0]) == [0, -3, -3] and list(p[1]) == [1, -3, -3]
    assert list(p[2]) == [3, 4, -3] and list(p[3]) == [2, 5, -3] and list(p[4]) == [3, 6, -3]
    assert np.array_equal(bk2[1], bk[1])          # request 1 untouched
    # out of range: parent == W_old, step == T_cap, beam index >= W_cap
    len_full = np.array([0, 1, 3], dtype=np.int32)
    parent_bad = np.array([0, 0, 2, 0, 0], dtype=np.int32)
    p, ln, bk3, bv3, sk = fn(ro_old, ro_new, parent_bad, path_old, len_full, new_k, new_k,
                             path_init, bk, bv, W_cap)
    assert sk == 3, sk                              # request 2: step 3 == T_cap
    assert list(ln) == [1, 1, 4]
    assert np.array_equal(p[2:], path_init[2:])
    ro_wide = np.array([0, 5, 5, 5], dtype=np.int32)
    nk5 = rng.integers(0, 1 << 16, size=(5, Hkv, D), dtype=np.uint16)
    p, ln, bk4, _, sk = fn(ro_old, ro_wide, parent, path_old, np.zeros(3, np.int32), nk5, nk5,
                           path_init, bk, bv, W_cap)
    assert sk == 1                                   # beam 4 >= W_cap
    assert np.array_equal(bk4[0, 4:], bk[0, 4:])
    # parent == W_old at step 1
    parent_eq = np.array([0, 0, 2, 1, 0], dtype=np.int32)
    _, _, _, _, sk = fn(ro_old, ro_new, parent_eq, path_old, len_old, new_k, new_k, path_init,
                        bk, bv, W_cap)
    assert sk == 1
    # a negative parent at step 1 (request 2, beam 1)
    parent_neg = np.array([0, 0, 1, -1, 0], dtype=np.int32)
    p, _, bk5, _, sk = fn(ro_old, ro_new, parent_neg, path_old, len_old, new_k, new_k, path_init,
                          bk, bv, W_cap)
    assert sk == 1
    assert np.array_equal(p[3], path_init[3]) and list(p[4]) == [2, 6, -3]
    assert np.array_equal(bk5[2, 5], bk[2, 5])       # its slot keeps its contents
    # a BeamKV pool of 6 slots: request 2 at step 1 writes slots 4 + k, so its
    # beam 2 (slot 6) is out of range and writes nothing
    p, _, bk6, _, sk = fn(ro_old, ro_new, parent, path_old, len_old, new_k, new_k, path_init,
                          bk[:, :6].copy(), bv[:, :6].copy(), W_cap)
    assert sk == 1
    assert list(p[2]) == [3, 4, -3] and list(p[3]) == [2, 5, -3]
    assert np.array_equal(p[4], path_init[4])
    assert np.array_equal(bk6[2, 5], new_k[3]) and np.array_equal(bk6[0, :2], new_k[:2])


def battery(fn: StepFn) -> List[str]:
    """Names of the pins that reject ``fn`` (empty: all pass)."""
    failed = []
    for name, pin in (("P1", pin_p1_chain_walk), ("P2", pin_p2_append),
                      ("P3", pin_p3_composition), ("P4", pin_p4_special)):
        try:
            pin(fn)
        except (AssertionError, IndexError, ValueError, RuntimeError):
            failed.append(name)
    return failed
