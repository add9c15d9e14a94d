"""Independent checks that pin the fp64 oracle (not a test module itself).

Each ``pin_*`` takes an oracle callable with the signature of
``oracle.decode_attn`` and raises ``AssertionError`` when the oracle disagrees
with something fixed by the mathematics or by a library routine:

* S1  plain attention: one beam, no beam tokens == torch SDPA (fp64)
* S2  per-row concatenation: context ++ BeamKV tokens found by walking the
      parent chains (not the resolved BeamPath table) == torch SDPA (fp64)
* S3  brute force at 50 significant digits (mpmath) on tiny inputs
* S4  closed forms: q = 0; all values equal; a single key; no key at all
* S5  permuting a request's rows permutes the outputs bitwise
* S6  rows with identical (q, path) give bitwise identical outputs
* S7  log-sum-exp algebra: merging context-only and path-only results
      reproduces the full result
* S8  GQA: grouped heads == the same heads with K/V repeated explicitly
* NaN padding never reaches the outputs

The tolerances are far below bf16 resolution; they only absorb fp64 rounding
differences between summation orders.
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

from shared_prefix_beam_amd import inputs as I

OracleFn = Callable[..., tuple]


def call(fn: OracleFn, inp: I.Inputs, rows=None, scale=None):
    return fn(inp.q, inp.ctx_k, inp.ctx_v, inp.ctx_len, inp.beam_k, inp.beam_v,
              inp.beam_path, inp.beam_len, inp.row_offset,
              scale=inp.scale if scale is None else scale, rows=rows)


def f64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def chain_slots(inp: I.Inputs, r: int) -> List[int]:
    """BeamKV slots on row r's path, found by walking parent pointers from
    the row's own current slot back to step 0 (independent of beam_path)."""
    b = int(np.searchsorted(inp.row_offset, r, side="right") - 1)
    w = r - int(inp.row_offset[b])
    if inp.dup_src[b] is not None and w in set(int(x) for x in inp.dup_rows[b]):
        w = inp.dup_src[b]
    T = int(inp.beam_len[b])
    slots = []
    k = w
    for s in range(T - 1, -1, -1):
        slots.append(s * inp.W_cap + k)
        if s > 0:
            k = int(inp.parents[b][s][k])
    return slots[::-1]


def concat_kv(inp: I.Inputs, r: int, g: int):
    b = int(np.searchsorted(inp.row_offset, r, side="right") - 1)
    L = int(inp.ctx_len[b])
    slots = chain_slots(inp, r)
    K = np.concatenate([f64(inp.ctx_k[b, :L, g]), f64(inp.beam_k[b, slots, g])], axis=0)
    V = np.concatenate([f64(inp.ctx_v[b, :L, g]), f64(inp.beam_v[b, slots, g])], axis=0)
    return K, V


def sdpa_row(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """torch SDPA (math path, fp64 CPU) for one query vector; plus logsumexp."""
    qt = torch.from_numpy(q_row).view(1, 1, 1, -1)
    Kt = torch.from_numpy(K).view(1, 1, K.shape[0], -1)
    Vt = torch.from_numpy(V).view(1, 1, V.shape[0], -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    lse = torch.logsumexp((torch.from_numpy(K) @ torch.from_numpy(q_row)) * scale, dim=0)
    return o.view(-1).numpy(), float(lse)


# ---------------------------------------------------------------------------
def pin_s1_plain_attention(fn: OracleFn, seed: int = 7):
    """One request, one beam, no beam tokens, G = 2: equals SDPA with enable_gqa."""
    inp = I.custom(B=1, Hq=4, Hkv=2, D=32, W=[1], ctx_len=[37], beam_len=[0], seed=seed)
    out, lse = call(fn, inp)
    q = torch.from_numpy(f64(inp.q)).permute(1, 0, 2).unsqueeze(0)         # [1,Hq,1,D]
    K = torch.from_numpy(f64(inp.ctx_k[0, :37])).permute(1, 0, 2).unsqueeze(0)  # [1,Hkv,L,D]
    V = torch.from_numpy(f64(inp.ctx_v[0, :37])).permute(1, 0, 2).unsqueeze(0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=inp.scale,
                                                           enable_gqa=True)
    ref = ref[0, :, 0, :].numpy()
    Kr = K.repeat_interleave(2, dim=1)
    ref_lse = torch.logsumexp((q @ Kr.transpose(-1, -2))[0, :, 0, :] * inp.scale, dim=-1).numpy()
    assert np.max(np.abs(out[0] - ref)) < 1e-12, "S1 out"
    assert np.max(np.abs(lse[0] - ref_lse)) < 1e-12, "S1 lse"


def pin_s2_concatenation(fn: OracleFn, inp: I.Inputs, rows: Sequence[int]):
    """Sampled rows: explicit context ++ chain-walked beam tokens, SDPA fp64."""
    rows = list(rows)
    out, lse = call(fn, inp, rows=rows)
    G = inp.wl.G
    for i, r in enumerate(rows):
        for h in range(inp.wl.Hq):
            K, V = concat_kv(inp, r, h // G)
            ref, ref_lse = sdpa_row(f64(inp.q[r, h]), K, V, inp.scale)
            assert np.max(np.abs(out[i, h] - ref)) < 1e-12, f"S2 out row {r} head {h}"
            assert abs(lse[i, h] - ref_lse) < 1e-12, f"S2 lse row {r} head {h}"


def pin_s3_bruteforce(fn: OracleFn, inp: I.Inputs, rows: Optional[Sequence[int]] = None):
    """mpmath at 50 digits, chain-walked keys."""
    import mpmath
    mpmath.mp.dps = 50
    rows = list(range(inp.R)) if rows is None else list(rows)
    out, lse = call(fn, inp, rows=rows)
    G = inp.wl.G
    scale = mpmath.mpf(1) / mpmath.sqrt(inp.wl.D)
    for i, r in enumerate(rows):
        for h in range(inp.wl.Hq):
            K, V = concat_kv(inp, r, h // G)
            q = [mpmath.mpf(float(x)) for x in f64(inp.q[r, h])]
            if K.shape[0] == 0:
                assert lse[i, h] == -math.inf and np.all(out[i, h] == 0), "S3 empty"
                continue
            z = [scale * mpmath.fsum(q[d] * mpmath.mpf(float(K[j, d])) for d in range(len(q)))
                 for j in range(K.shape[0])]
            e = [mpmath.exp(x) for x in z]
            Z = mpmath.fsum(e)
            ref_lse = mpmath.log(Z)
            for d in range(V.shape[1]):
                ref = mpmath.fsum(e[j] * mpmath.mpf(float(V[j, d])) for j in range(K.shape[0])) / Z
                assert abs(out[i, h, d] - float(ref)) < 1e-13, f"S3 out row {r} head {h} d {d}"
            assert abs(lse[i, h] - float(ref_lse)) < 1e-13, f"S3 lse row {r} head {h}"


def pin_s4_closed_forms(fn: OracleFn, seed: int = 11):
    # (a) q = 0: every score is 0, so lse = ln N and out = mean of the N values
    inp = I.custom(B=2, Hq=2, Hkv=1, D=16, W=[3, 2], ctx_len=[5, 9], beam_len=[2, 3], seed=seed)
    inp.q[:] = 0
    out, lse = call(fn, inp)
    for r in range(inp.R):
        b = int(np.searchsorted(inp.row_offset, r, side="right") - 1)
        N = int(inp.ctx_len[b] + inp.beam_len[b])
        K, V = concat_kv(inp, r, 0)
        assert np.all(np.abs(lse[r] - math.log(N)) <= 1e-15), "S4a lse = ln N"
        assert np.max(np.abs(out[r] - V.mean(axis=0))) < 1e-14, "S4a out = mean V"
    # (b) every value row equal to one vector c: out = c
    inp = I.custom(B=2, Hq=4, Hkv=2, D=16, W=[2, 3], ctx_len=[6, 4], beam_len=[3, 1], seed=seed + 1)
    c = inp.ctx_v[0, 0, 0].copy()
    for arr, lens in ((inp.ctx_v, inp.ctx_len), (inp.beam_v, None)):
        for b in range(inp.B):
            if lens is None:
                arr[b, :-1] = c          # all live slots (the last slot stays NaN padding)
            else:
                arr[b, :int(lens[b])] = c
    out, _ = call(fn, inp)
    assert np.max(np.abs(out - f64(c)[None, None, :]) / (np.abs(f64(c)) + 1e-300)) < 1e-14, "S4b"
    # (c) a single key: out = its value, lse = its score
    for L, T in ((1, 0), (0, 1)):
        inp = I.custom(B=1, Hq=2, Hkv=1, D=8, W=[2], ctx_len=[L], beam_len=[T], seed=seed + 2,
                       ctx_cap=2, T_cap=2)
        out, lse = call(fn, inp)
        for r in range(inp.R):
            K, V = concat_kv(inp, r, 0)
            for h in range(2):
                z0 = inp.scale * float(np.dot(f64(inp.q[r, h]), K[0]))
                assert np.all(out[r, h] == V[0]), "S4c out = V0"
                assert abs(lse[r, h] - z0) < 1e-15, "S4c lse = z0"
    # (d) no key at all: out = 0, lse = -inf
    inp = I.custom(B=1, Hq=2, Hkv=1, D=8, W=[2], ctx_len=[0], beam_len=[0], seed=seed + 3,
                   ctx_cap=2, T_cap=2)
    out, lse = call(fn, inp)
    assert np.all(out == 0) and np.all(lse == -np.inf), "S4d empty"


def pin_s5_permutation(fn: OracleFn, inp: I.Inputs, seed: int = 5):
    """Permute each request's rows (q and path together): outputs permute bitwise."""
    out, lse = call(fn, inp)
    rng = np.random.default_rng(seed)
    perm = np.arange(inp.R)
    for b in range(inp.B):
        r0, r1 = int(inp.row_offset[b]), int(inp.row_offset[b + 1])
        perm[r0:r1] = r0 + rng.permutation(r1 - r0)
    q2 = inp.q[perm].copy()
    p2 = inp.beam_path[perm].copy()
    out2, lse2 = fn(q2, inp.ctx_k, inp.ctx_v, inp.ctx_len, inp.beam_k, inp.beam_v, p2,
                    inp.beam_len, inp.row_offset, scale=inp.scale)
    assert np.array_equal(out2, out[perm]) and np.array_equal(lse2, lse[perm]), "S5"


def pin_s6_duplicates(fn: OracleFn, inp: I.Inputs):
    """Give duplicate-path rows their source's q: outputs must match bitwise."""
    q = inp.q.copy()
    pairs = []
    for b in range(inp.B):
        if inp.dup_src[b] is None:
            continue
        r0 = int(inp.row_offset[b])
        src = r0 + inp.dup_src[b]
        for w in inp.dup_rows[b][:8]:
            q[r0 + int(w)] = q[src]
            pairs.append((src, r0 + int(w)))
    assert pairs, "S6 needs duplicate-path rows"
    out, lse = fn(q, inp.ctx_k, inp.ctx_v, inp.ctx_len, inp.beam_k, inp.beam_v, inp.beam_path,
                  inp.beam_len, inp.row_offset, scale=inp.scale,
                  rows=[x for p in pairs for x in p])
    for i in range(len(pairs)):
        assert np.array_equal(out[2 * i], out[2 * i + 1]), "S6 out"
        assert np.array_equal(lse[2 * i], lse[2 * i + 1]), "S6 lse"


def pin_s7_lse_merge(fn: OracleFn, inp: I.Inputs, rows: Sequence[int]):
    """context-only (beam_len = 0) and path-only (ctx_len = 0) results, merged by
    log-sum-exp weights, reproduce the result over both key sets."""
    rows = list(rows)
    out, lse = call(fn, inp, rows=rows)
    zeros = np.zeros_like(inp.ctx_len)
    oc, lc = fn(inp.q, inp.ctx_k, inp.ctx_v, inp.ctx_len, inp.beam_k, inp.beam_v,
                inp.beam_path, zeros, inp.row_offset, scale=inp.scale, rows=rows)
    ou, lu = fn(inp.q, inp.ctx_k, inp.ctx_v, zeros, inp.beam_k, inp.beam_v,
                inp.beam_path, inp.beam_len, inp.row_offset, scale=inp.scale, rows=rows)
    m = np.maximum(lc, lu)
    wc = np.exp(lc - m)
    wu = np.exp(lu - m)
    merged = (wc[..., None] * oc + wu[..., None] * ou) / (wc + wu)[..., None]
    mlse = m + np.log(wc + wu)
    assert np.max(np.abs(merged - out)) < 1e-13, "S7 out"
    assert np.max(np.abs(mlse - lse)) < 1e-13, "S7 lse"


def pin_s8_gqa(fn: OracleFn, seed: int = 13):
    """G = 4 grouped heads equal Hkv = Hq with every KV head repeated G times."""
    inp = I.custom(B=2, Hq=8, Hkv=2, D=16, W=[3, 2], ctx_len=[7, 5], beam_len=[2, 3], seed=seed)
    out, lse = call(fn, inp)
    G = 4
    rk = lambda a: np.repeat(a, G, axis=2)
    out2, lse2 = fn(inp.q, rk(inp.ctx_k), rk(inp.ctx_v), inp.ctx_len, rk(inp.beam_k),
                    rk(inp.beam_v), inp.beam_path, inp.beam_len, inp.row_offset, scale=inp.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "S8"


def pin_nan_padding(fn: OracleFn, inp: I.Inputs, rows=None):
    out, lse = call(fn, inp, rows=rows)
    assert np.isfinite(out).all() and np.isfinite(lse).all(), "NaN padding leaked"


def tiny_cases(n: int = 6, seed: int = 1000) -> List[I.Inputs]:
    """Random tiny shapes: L <= 8, T <= 3, W <= 4, D = 4, G in {1, 2}."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.integers(1, 3))
        W = [int(x) for x in rng.integers(1, 5, size=B)]
        L = [int(x) for x in rng.integers(0, 9, size=B)]
        T = [int(x) for x in rng.integers(0, 4, size=B)]
        cases.append(I.custom(B=B, Hq=G * Hkv, Hkv=Hkv, D=4, W=W, ctx_len=L, beam_len=T,
                              seed=seed + i, ctx_cap=8, T_cap=3, grow_steps=bool(i % 2)))
    return cases


def sharp_case(seed: int = 31) -> I.Inputs:
    """Scores in the hundreds to thousands: exp overflows unless the true
    maximum is subtracted first."""
    return I.custom(B=2, Hq=2, Hkv=1, D=4, W=[3, 2], ctx_len=[8, 5], beam_len=[2, 3],
                    seed=seed, q_std=1000.0)


def battery(fn: OracleFn, quick: bool = True) -> List[str]:
    """Run every pin on small inputs; return the names of the pins that fail."""
    failed = []
    c1 = I.generate(I.WORKLOADS[1])
    dup = I.custom(B=2, Hq=4, Hkv=2, D=16, W=[6, 5], ctx_len=[9, 4], beam_len=[3, 2],
                   seed=21, dup_frac=0.5)
    rag = I.custom(B=3, Hq=4, Hkv=2, D=16, W=[3, 5, 2], ctx_len=[12, 0, 7], beam_len=[2, 3, 0],
                   seed=22, ctx_cap=16, T_cap=4, grow_steps=True)
    checks = [
        ("S1", lambda: pin_s1_plain_attention(fn)),
        ("S2", lambda: pin_s2_concatenation(fn, rag, range(rag.R))),
        ("S2c1", lambda: pin_s2_concatenation(fn, c1, range(c1.R))),
        ("S3", lambda: [pin_s3_bruteforce(fn, c) for c in tiny_cases(3 if quick else 8)]),
        ("S3sharp", lambda: pin_s3_bruteforce(fn, sharp_case())),
        ("S4", lambda: pin_s4_closed_forms(fn)),
        ("S5", lambda: pin_s5_permutation(fn, dup)),
        ("S6", lambda: pin_s6_duplicates(fn, dup)),
        ("S7", lambda: pin_s7_lse_merge(fn, rag, range(rag.R))),
        ("S8", lambda: pin_s8_gqa(fn)),
        ("NaN", lambda: pin_nan_padding(fn, rag)),
    ]
    for name, f in checks:
        try:
            with np.errstate(all="ignore"):
                f()
        except (AssertionError, RuntimeError, IndexError, ValueError) as e:
            failed.append(f"{name}: {e}")
    return failed
