"""Helpers for the GPU tests: device upload, running the library, comparing
against the oracle with the parity tolerances."""
from __future__ import annotations

import numpy as np

from shared_prefix_beam_amd import inputs as I

# parity tolerances (bf16 outputs, fp32 natural-log LSE)
MAX_ABS = 2e-2
MAX_REL = 1e-2      # row-wise: max_d |gpu - ref| / max_d |ref|, per (row, head)
LSE_ABS = 1e-3


def log(msg: str):
    print(msg, flush=True)


def run_lib(inp: I.Inputs, which: str = "fused", dev=None, scale=None, tiling=None):
    """Run the library on ``inp``; return (out float32 numpy [R,Hq,D], lse numpy [R,Hq]).
    ``tiling`` = (nqt, nks[, n_split]) forces the fused kernel's work decomposition."""
    import torch
    from shared_prefix_beam_amd import gr_attn
    t = dev if dev is not None else I.to_torch(inp)
    kw = dict(tiling=tiling) if which == "fused" else {}
    fn = gr_attn.decode_attn if which == "fused" else gr_attn.decode_attn_generic
    out, lse = fn(t["q"], t["ctx_k"], t["ctx_v"], t["ctx_len"], t["beam_k"], t["beam_v"],
                  t["beam_path"], t["beam_len"], t["row_offset"], W_max=int(max(inp.wl.W)),
                  scale=scale, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def errors(out, lse, ref_out, ref_lse):
    """(max abs, max row-wise rel, max lse abs) between device and oracle results."""
    d = np.abs(out.astype(np.float64) - ref_out)
    max_abs = float(d.max()) if d.size else 0.0
    denom = np.abs(ref_out).max(axis=-1)
    rel = d.max(axis=-1) / np.where(denom > 0, denom, 1.0)
    max_rel = float(rel.max()) if rel.size else 0.0
    fin = np.isfinite(ref_lse)
    lse_err = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    assert np.array_equal(np.isfinite(lse), fin), "LSE finiteness differs"
    return max_abs, max_rel, lse_err


def assert_parity(out, lse, ref_out, ref_lse, what=""):
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    a, r, l = errors(out, lse, ref_out, ref_lse)
    log(f"  {what}: max_abs={a:.3e} max_rel={r:.3e} lse_abs={l:.3e}")
    assert a <= MAX_ABS, f"{what}: max abs {a}"
    assert r <= MAX_REL, f"{what}: max rel {r}"
    assert l <= LSE_ABS, f"{what}: lse abs {l}"
