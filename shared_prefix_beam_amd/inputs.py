"""Seeded synthetic inputs for large-beam decode attention.

This module only draws inputs: random bf16 tensors, ragged lengths, beam
parent chains and the resolved BeamPath table.  It holds none of the attention
arithmetic, so both the HIP path and the CPU oracle can take their inputs from
here without sharing any of the method.

Data model (GR-Inference blog, section on system design; xGR review, section
"xAttention", KV cache management):

* ContextKV: one long prefill KV per request, shared by all of its beams.
  Layout ``[B][ctx_cap][Hkv][D]`` bf16; tokens ``j >= ctx_len[b]`` are padding.
* BeamKV: the short per-beam KV written during decode, one token per
  (step, live beam).  Layout ``[B][beam_cap][Hkv][D]`` bf16, step-major:
  step ``s``, beam slot ``k`` lives at flat index ``s * W_cap + k``.  One extra
  slot at index ``T_cap * W_cap`` is always padding; unused BeamPath entries
  point at it.
* BeamPath: for each query row (one live beam of one request) the flat BeamKV
  indices of the tokens on its ancestry chain, step 0 first, its own current
  token last.  Layout ``[R][T_cap]`` int32; entries ``s >= beam_len[b]`` are
  padding.
* Rows of all requests are packed: request ``b`` owns rows
  ``row_offset[b] .. row_offset[b+1]-1``; q is ``[R][Hq][D]`` bf16.

Every padding element of every bf16 buffer is a quiet NaN, so a kernel that
reads outside the valid region produces NaN in its output.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic decode-attention call."""

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    W: Sequence[int]            # beams (query rows) per request
    ctx: tuple                  # ("fixed", L) or ("uniform", lo, hi), inclusive
    T: tuple                    # ("fixed", T) or ("uniform", lo, hi), inclusive
    seed: int
    q_std: float = 1.0
    kv_std: float = 1.0
    dup_frac: float = 0.0       # fraction of beams that copy one beam's full path row
    grow_steps: bool = False    # per-step beam width grows from W/8 to W

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The five workloads: Qwen3 attention shapes (0.6B/1.7B: Hq=16, Hkv=8;
# 4B: Hq=32, Hkv=8; head dim 128), contexts of 1k-4k tokens, beam widths
# 4-900 and 2-5 decode tokens, as on the GR-Inference and SID-GR pages.
WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny_b1_l64_w4_g2_d64", B=1, Hq=2, Hkv=1, D=64, W=(4,),
                ctx=("fixed", 64), T=("fixed", 3), seed=101),
    2: Workload("qwen3_0.6b_b8_l1024_w128", B=8, Hq=16, Hkv=8, D=128, W=(128,) * 8,
                ctx=("fixed", 1024), T=("fixed", 3), seed=202),
    3: Workload("qwen3_1.7b_b16_l512-4096_w256_ragged", B=16, Hq=16, Hkv=8, D=128,
                W=(256,) * 16, ctx=("uniform", 512, 4096), T=("uniform", 2, 5),
                seed=303, q_std=0.5),
    4: Workload("qwen3_0.6b_b4_l2048_w900_dup30", B=4, Hq=16, Hkv=8, D=128,
                W=(900,) * 4, ctx=("fixed", 2048), T=("fixed", 3), seed=404,
                dup_frac=0.3),
    5: Workload("qwen3_4b_b6_l1024-3072_w20-900_grow", B=6, Hq=32, Hkv=8, D=128,
                W=(20, 128, 256, 512, 512, 900), ctx=("uniform", 1024, 3072),
                T=("fixed", 5), seed=505, grow_steps=True),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); return raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def step_widths(W: int, T: int, grow: bool) -> List[int]:
    """Live beams at each decode step s = 0..T-1; the last step has W beams.

    With ``grow`` the width rises linearly from W/8 at step 0 to W at the last
    step (floor, at least 1); otherwise every step has W beams.
    """
    if not grow or T <= 1:
        return [W] * T
    return [max(1, (W * (T - 1 + 7 * s)) // (8 * (T - 1))) for s in range(T)]


@dataclasses.dataclass
class Inputs:
    """One generated call.  bf16 tensors are uint16 bit patterns."""

    wl: Workload
    q: np.ndarray           # [R][Hq][D] u16
    ctx_k: np.ndarray       # [B][ctx_cap][Hkv][D] u16
    ctx_v: np.ndarray
    beam_k: np.ndarray      # [B][beam_cap][Hkv][D] u16
    beam_v: np.ndarray
    ctx_len: np.ndarray     # [B] i32
    beam_len: np.ndarray    # [B] i32
    row_offset: np.ndarray  # [B+1] i32
    beam_path: np.ndarray   # [R][T_cap] i32
    widths: List[List[int]]                 # per request, per step live beams
    parents: List[List[np.ndarray]]         # per request, per step s>=1: parent slot of each slot
    dup_src: List[Optional[int]]            # per request: beam whose path row was copied
    dup_rows: List[np.ndarray]              # per request: beams that copied it
    W_cap: int
    T_cap: int

    @property
    def B(self) -> int:
        return self.wl.B

    @property
    def R(self) -> int:
        return int(self.row_offset[-1])

    @property
    def ctx_cap(self) -> int:
        return self.ctx_k.shape[1]

    @property
    def beam_cap(self) -> int:
        return self.beam_k.shape[1]

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.wl.D))

    def arrays(self) -> Dict[str, np.ndarray]:
        return dict(q=self.q, ctx_k=self.ctx_k, ctx_v=self.ctx_v, beam_k=self.beam_k,
                    beam_v=self.beam_v, ctx_len=self.ctx_len, beam_len=self.beam_len,
                    row_offset=self.row_offset, beam_path=self.beam_path)

    def digest(self) -> str:
        """SHA-256 over every buffer, to pin generator reproducibility."""
        h = hashlib.sha256()
        for k, v in self.arrays().items():
            h.update(k.encode())
            h.update(np.ascontiguousarray(v).tobytes())
        return h.hexdigest()


def _draw_len(rng: np.random.Generator, spec: tuple, B: int) -> np.ndarray:
    if spec[0] == "fixed":
        return np.full(B, spec[1], dtype=np.int32)
    lo, hi = spec[1], spec[2]
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def _cap(spec: tuple) -> int:
    return spec[1] if spec[0] == "fixed" else spec[2]


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_bits(x)


def generate(wl: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw one call of workload ``wl``.

    Draw order is fixed: lengths, q, ctx_k, ctx_v, beam_k, beam_v, parent
    chains, duplicate-path choices.  Padding is poisoned with bf16 NaN after
    all draws, so the valid values do not depend on the padding.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    ctx_len = _draw_len(rng, wl.ctx, wl.B)
    beam_len = _draw_len(rng, wl.T, wl.B)
    return _build(rng, wl, ctx_len, beam_len, _cap(wl.ctx), _cap(wl.T))


def custom(B: int, Hq: int, Hkv: int, D: int, W: Sequence[int], ctx_len: Sequence[int],
           beam_len: Sequence[int], seed: int, ctx_cap: Optional[int] = None,
           T_cap: Optional[int] = None, q_std: float = 1.0, grow_steps: bool = False,
           dup_frac: float = 0.0, W_cap: Optional[int] = None) -> Inputs:
    """Inputs with explicit per-request lengths (edge cases, small parity shapes)."""
    ctx_len = np.asarray(ctx_len, dtype=np.int32)
    beam_len = np.asarray(beam_len, dtype=np.int32)
    ctx_cap = max(int(ctx_len.max()), 1) if ctx_cap is None else ctx_cap
    T_cap = max(int(beam_len.max()), 1) if T_cap is None else T_cap
    wl = Workload(f"custom_s{seed}", B=B, Hq=Hq, Hkv=Hkv, D=D, W=tuple(W),
                  ctx=("fixed", ctx_cap), T=("fixed", T_cap), seed=seed, q_std=q_std,
                  grow_steps=grow_steps, dup_frac=dup_frac)
    return _build(np.random.default_rng(seed), wl, ctx_len, beam_len, ctx_cap, T_cap, W_cap)


def _build(rng: np.random.Generator, wl: Workload, ctx_len: np.ndarray,
           beam_len: np.ndarray, ctx_cap: int, T_cap: int,
           W_cap: Optional[int] = None) -> Inputs:
    B, Hq, Hkv, D = wl.B, wl.Hq, wl.Hkv, wl.D
    assert Hq % Hkv == 0 and len(wl.W) == B
    assert int(ctx_len.max(initial=0)) <= ctx_cap and int(beam_len.max(initial=0)) <= T_cap
    W = np.asarray(wl.W, dtype=np.int64)
    row_offset = np.zeros(B + 1, dtype=np.int32)
    row_offset[1:] = np.cumsum(W)
    R = int(row_offset[-1])
    W_cap = max(int(W.max(initial=0)), 1) if W_cap is None else int(W_cap)
    assert W_cap >= int(W.max(initial=0))
    beam_cap = T_cap * W_cap + 1          # + one always-padding slot
    pad_slot = T_cap * W_cap

    q = _normal_bf16(rng, (R, Hq, D), wl.q_std)
    ctx_k = _normal_bf16(rng, (B, ctx_cap, Hkv, D), wl.kv_std)
    ctx_v = _normal_bf16(rng, (B, ctx_cap, Hkv, D), wl.kv_std)
    beam_k = _normal_bf16(rng, (B, beam_cap, Hkv, D), wl.kv_std)
    beam_v = _normal_bf16(rng, (B, beam_cap, Hkv, D), wl.kv_std)

    beam_path = np.full((R, T_cap), pad_slot, dtype=np.int32)
    widths: List[List[int]] = []
    parents: List[List[np.ndarray]] = []
    for b in range(B):
        T = int(beam_len[b])
        ws = step_widths(int(W[b]), T, wl.grow_steps)
        widths.append(ws)
        par = [np.zeros(0, dtype=np.int64)]
        for s in range(1, T):
            par.append(rng.integers(0, ws[s - 1], size=ws[s]))
        parents.append(par)
        # walk every final beam back to step 0 (vectorised over beams)
        k = np.arange(W[b], dtype=np.int64)
        rows = beam_path[row_offset[b]:row_offset[b + 1]]
        for s in range(T - 1, -1, -1):
            rows[:, s] = s * W_cap + k
            if s > 0:
                k = par[s][k]

    dup_src: List[Optional[int]] = []
    dup_rows: List[np.ndarray] = []
    for b in range(B):
        Wb = int(W[b])
        n_dup = min(int(round(wl.dup_frac * Wb)), max(Wb - 1, 0))
        if n_dup == 0:
            dup_src.append(None)
            dup_rows.append(np.zeros(0, dtype=np.int64))
            continue
        src = int(rng.integers(0, Wb))
        others = np.delete(np.arange(Wb), src)
        sel = np.sort(rng.choice(others, size=n_dup, replace=False))
        r0 = int(row_offset[b])
        beam_path[r0 + sel] = beam_path[r0 + src]
        dup_src.append(src)
        dup_rows.append(sel)

    # poison padding
    for b in range(B):
        ctx_k[b, ctx_len[b]:] = BF16_NAN
        ctx_v[b, ctx_len[b]:] = BF16_NAN
        live = np.zeros(beam_cap, dtype=bool)
        for s, ws in enumerate(widths[b]):
            live[s * W_cap: s * W_cap + ws] = True
        beam_k[b, ~live] = BF16_NAN
        beam_v[b, ~live] = BF16_NAN

    return Inputs(wl=wl, q=q, ctx_k=ctx_k, ctx_v=ctx_v, beam_k=beam_k, beam_v=beam_v,
                  ctx_len=np.asarray(ctx_len, dtype=np.int32),
                  beam_len=np.asarray(beam_len, dtype=np.int32), row_offset=row_offset,
                  beam_path=beam_path, widths=widths, parents=parents,
                  dup_src=dup_src, dup_rows=dup_rows, W_cap=W_cap, T_cap=T_cap)


@dataclasses.dataclass
class PagedCtx:
    """A call's ContextKV scattered over fixed-size pages of a shared pool."""

    k_pages: np.ndarray      # [n_pages][page_size][Hkv][D] u16
    v_pages: np.ndarray
    page_table: np.ndarray   # [B][pages_per_req] i32
    page_size: int


def to_paged(inp: Inputs, page_size: int, seed: int, spare: int = 3) -> PagedCtx:
    """Scatter ``inp``'s ContextKV over pages in a seeded random order.

    Request b's logical page j (tokens j*page_size ..) goes to a distinct
    physical page; ``spare`` extra pages and the rows past ctx_len are bf16
    NaN, and table entries past a request's last page point at a NaN page,
    so a kernel that reads a wrong page or row produces NaN."""
    rng = np.random.default_rng(seed)
    ppr = max(-(-inp.ctx_cap // page_size), 1)
    used = [max(-(-int(inp.ctx_len[b]) // page_size), 0) for b in range(inp.B)]
    n_pages = sum(used) + spare
    Hkv, D = inp.wl.Hkv, inp.wl.D
    k_pages = np.full((n_pages, page_size, Hkv, D), BF16_NAN, dtype=np.uint16)
    v_pages = np.full_like(k_pages, BF16_NAN)
    perm = rng.permutation(n_pages)
    table = np.empty((inp.B, ppr), dtype=np.int32)
    nxt = 0
    for b in range(inp.B):
        for j in range(ppr):
            if j < used[b]:
                pg = int(perm[nxt])
                nxt += 1
                lo = j * page_size
                hi = min(lo + page_size, int(inp.ctx_len[b]))
                k_pages[pg, :hi - lo] = inp.ctx_k[b, lo:hi]
                v_pages[pg, :hi - lo] = inp.ctx_v[b, lo:hi]
                table[b, j] = pg
            else:
                table[b, j] = int(perm[n_pages - 1 - (j % spare)]) if spare else 0
    return PagedCtx(k_pages=k_pages, v_pages=v_pages, page_table=table, page_size=page_size)


@dataclasses.dataclass
class StepInputs:
    """One BeamKV-append + BeamPath-update call and the state it applies to.

    ``state`` holds the previous step's rows (``state.row_offset``), their
    paths of ``state.beam_len[b]`` tokens and the BeamKV caches, with room for
    one more step.  Beam selection produced ``row_offset_new`` new rows; new
    row r descends from old beam ``parent[r]`` of its request, and its
    current token's K/V (all KV heads) are ``new_k[r]``, ``new_v[r]``.
    """

    state: Inputs
    row_offset_new: np.ndarray  # [B+1] i32
    parent: np.ndarray          # [R_new] i32, in [0, W_old_b) (0 where the paths are empty)
    new_k: np.ndarray           # [R_new][Hkv][D] u16
    new_v: np.ndarray

    @property
    def R_new(self) -> int:
        return int(self.row_offset_new[-1])

    def digest(self) -> str:
        h = hashlib.sha256(self.state.digest().encode())
        for a in (self.row_offset_new, self.parent, self.new_k, self.new_v):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def step_inputs(B: int, Hkv: int, D: int, W_old: Sequence[int], W_new: Sequence[int],
                beam_len: Sequence[int], seed: int, T_cap: Optional[int] = None,
                W_cap: Optional[int] = None, Hq: Optional[int] = None) -> StepInputs:
    """A seeded beam-step call.  The state is drawn as ``custom`` draws a
    call (context of one token, which the step does not read), with T_cap at
    least beam_len + 1 and W_cap at least every width; then parents (uniform
    over the request's old beams) and the new K/V rows, in that order."""
    beam_len = np.asarray(beam_len, dtype=np.int32)
    T_cap = int(beam_len.max(initial=0)) + 1 if T_cap is None else T_cap
    W_cap = max(max(W_old, default=1), max(W_new, default=1), 1) if W_cap is None else W_cap
    state = custom(B=B, Hq=Hkv if Hq is None else Hq, Hkv=Hkv, D=D, W=W_old,
                   ctx_len=[1] * B, beam_len=beam_len, seed=seed, T_cap=T_cap, W_cap=W_cap)
    rng = np.random.default_rng(seed + 7919)
    row_offset_new = np.zeros(B + 1, dtype=np.int32)
    row_offset_new[1:] = np.cumsum(np.asarray(W_new, dtype=np.int64))
    parent = np.zeros(int(row_offset_new[-1]), dtype=np.int32)
    for b in range(B):
        n = int(W_new[b])
        if n and int(beam_len[b]) > 0 and int(W_old[b]) > 0:
            parent[row_offset_new[b]:row_offset_new[b + 1]] = rng.integers(0, int(W_old[b]), size=n)
    R_new = int(row_offset_new[-1])
    new_k = _normal_bf16(rng, (R_new, Hkv, D), 1.0)
    new_v = _normal_bf16(rng, (R_new, Hkv, D), 1.0)
    return StepInputs(state=state, row_offset_new=row_offset_new, parent=parent,
                      new_k=new_k, new_v=new_v)


# Beam-step calls at the attention workloads' shapes: the step that appends
# token 3 to every request of the W=128 and W=900 workloads.
STEP_WORKLOADS = {
    2: dict(name="qwen3_0.6b_b8_w128_step3", B=8, Hkv=8, D=128, W_old=(128,) * 8,
            W_new=(128,) * 8, beam_len=(3,) * 8, seed=2202),
    4: dict(name="qwen3_0.6b_b4_w900_step3", B=4, Hkv=8, D=128, W_old=(900,) * 4,
            W_new=(900,) * 4, beam_len=(3,) * 4, seed=4404),
}


def step_workload(cfg: int) -> StepInputs:
    w = dict(STEP_WORKLOADS[cfg])
    w.pop("name")
    return step_inputs(**w)


@dataclasses.dataclass
class SelectInputs:
    """One beam-selection call: the previous step's beams and their next-token
    logits, and how many beams each request keeps."""

    row_offset_old: np.ndarray  # [B+1] i32
    row_offset_new: np.ndarray  # [B+1] i32 (request b keeps W_new[b] beams)
    score_old: np.ndarray       # [R_old] f32, cumulative log-probability of each beam
    logits: np.ndarray          # [R_old][V] f32

    @property
    def V(self) -> int:
        return self.logits.shape[1]


def select_inputs(W_old: Sequence[int], W_new: Sequence[int], V: int, seed: int,
                  logit_std: float = 2.0, score_spread: float = 3.0) -> SelectInputs:
    """Seeded selection call: cumulative scores -|N(0, score_spread)| (log
    probabilities), logits N(0, logit_std) in fp32; scores then logits."""
    rng = np.random.default_rng(seed)
    ro = np.zeros(len(W_old) + 1, dtype=np.int32)
    ro[1:] = np.cumsum(np.asarray(W_old, dtype=np.int64))
    rn = np.zeros(len(W_new) + 1, dtype=np.int32)
    rn[1:] = np.cumsum(np.asarray(W_new, dtype=np.int64))
    R = int(ro[-1])
    score = -np.abs(rng.standard_normal(R).astype(np.float32) * np.float32(score_spread))
    logits = rng.standard_normal((R, V), dtype=np.float32) * np.float32(logit_std)
    return SelectInputs(row_offset_old=ro, row_offset_new=rn, score_old=score, logits=logits)


# Beam selection at the attention workloads' widths, over an 8192-entry
# semantic-ID vocabulary.
SELECT_WORKLOADS = {
    2: dict(name="w128_b8_v8192", W_old=(128,) * 8, W_new=(128,) * 8, V=8192, seed=2303),
    4: dict(name="w900_b4_v8192", W_old=(900,) * 4, W_new=(900,) * 4, V=8192, seed=4505),
}


def select_workload(cfg: int) -> SelectInputs:
    w = dict(SELECT_WORKLOADS[cfg])
    w.pop("name")
    return select_inputs(**w)


def unique_beam_rows(inp: Inputs) -> List[int]:
    """Per request: number of distinct BeamKV tokens referenced by its paths."""
    out = []
    for b in range(inp.B):
        r0, r1 = int(inp.row_offset[b]), int(inp.row_offset[b + 1])
        T = int(inp.beam_len[b])
        out.append(int(np.unique(inp.beam_path[r0:r1, :T]).size) if T > 0 else 0)
    return out


def to_torch(inp: Inputs, device="cuda"):
    """Copy the generated buffers to ``device`` as torch tensors (bf16 / int32).

    Returns a dict with the entry-point argument names.
    """
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    return dict(q=bf(inp.q), ctx_k=bf(inp.ctx_k), ctx_v=bf(inp.ctx_v), ctx_len=i32(inp.ctx_len),
                beam_k=bf(inp.beam_k), beam_v=bf(inp.beam_v), beam_path=i32(inp.beam_path),
                beam_len=i32(inp.beam_len), row_offset=i32(inp.row_offset))


# ---- item catalog and its semantic-ID trie (constrained selection) ----------
@dataclasses.dataclass
class SidTrie:
    """A catalog of items, each a sequence of `depth` semantic-ID tokens in
    [0, V), and its prefix trie in CSR form (GR-Inference blog, kernel design:
    the SID trie kept in device memory as CSR).

    Node 0 is the root (the empty prefix); the nodes of prefix length d are
    numbered after those of length d-1, in lexicographic order of their
    prefixes.  Node u's children are edges node_ptr[u] .. node_ptr[u+1]-1,
    edge e carrying token edge_tok[e] (increasing within a node) to node
    edge_child[e]."""

    items: np.ndarray       # [N][depth] i32, distinct, lexicographically sorted
    node_ptr: np.ndarray    # [n_nodes + 1] i32
    edge_tok: np.ndarray    # [n_edges] i32
    edge_child: np.ndarray  # [n_edges] i32
    level_start: np.ndarray  # [depth + 2] i32: nodes of prefix length d are level_start[d] ..
    V: int

    @property
    def n_nodes(self) -> int:
        return int(self.node_ptr.size - 1)

    @property
    def n_edges(self) -> int:
        return int(self.edge_tok.size)

    def level_fanout(self, d: int) -> int:
        """Largest child count among the nodes of prefix length d."""
        f = np.diff(self.node_ptr)[self.level_start[d]:self.level_start[d + 1]]
        return int(f.max()) if f.size else 0

    def node_of(self, prefixes: np.ndarray) -> np.ndarray:
        """Node ids of prefixes [n][d] taken from the catalog (all of one
        length d); -1 for a prefix no item has."""
        prefixes = np.asarray(prefixes, dtype=np.int64).reshape(len(prefixes), -1)
        d = prefixes.shape[1]
        if d == 0:
            return np.zeros(len(prefixes), dtype=np.int32)
        codes = _prefix_codes(self.items[:, :d], self.V)
        uniq = np.unique(codes)
        q = _prefix_codes(prefixes, self.V)
        pos = np.searchsorted(uniq, q)
        pos_c = np.minimum(pos, uniq.size - 1)
        found = (pos < uniq.size) & (uniq[pos_c] == q)
        return np.where(found, self.level_start[d] + pos_c, -1).astype(np.int32)


def _prefix_codes(p: np.ndarray, V: int) -> np.ndarray:
    code = np.zeros(p.shape[0], dtype=np.int64)
    for j in range(p.shape[1]):
        code = code * V + p[:, j].astype(np.int64)
    return code


def sid_catalog(n_items: int, depth: int, V: int, seed: int) -> np.ndarray:
    """`n_items` distinct items of `depth` tokens, uniform in [0, V), sorted."""
    rng = np.random.default_rng(seed)
    items = rng.integers(0, V, size=(int(n_items * 1.05) + 16, depth), dtype=np.int64)
    items = np.unique(items, axis=0)
    if items.shape[0] > n_items:
        keep = np.sort(rng.choice(items.shape[0], size=n_items, replace=False))
        items = items[keep]
    return items.astype(np.int32)


def build_trie(items: np.ndarray, V: int) -> SidTrie:
    """CSR prefix trie of distinct, lexicographically sorted items."""
    items = np.asarray(items, dtype=np.int32)
    depth = items.shape[1]
    uniq = [np.zeros((1, 0), dtype=np.int32)]             # prefixes of each length
    for d in range(1, depth + 1):
        codes = _prefix_codes(items[:, :d], V)
        _, first = np.unique(codes, return_index=True)
        uniq.append(items[np.sort(first), :d])
    level_start = np.zeros(depth + 2, dtype=np.int64)
    for d in range(depth + 1):
        level_start[d + 1] = level_start[d] + uniq[d].shape[0]
    n_nodes = int(level_start[depth + 1])
    child_count = np.zeros(n_nodes, dtype=np.int64)
    edge_tok, edge_child = [], []
    for d in range(1, depth + 1):
        pre = uniq[d]
        parent_codes = _prefix_codes(pre[:, :d - 1], V)
        parent_pos = np.searchsorted(_prefix_codes(uniq[d - 1], V), parent_codes) \
            if d > 1 else np.zeros(pre.shape[0], dtype=np.int64)
        np.add.at(child_count, level_start[d - 1] + parent_pos, 1)
        edge_tok.append(pre[:, d - 1])
        edge_child.append(level_start[d] + np.arange(pre.shape[0]))
    node_ptr = np.zeros(n_nodes + 1, dtype=np.int64)
    node_ptr[1:] = np.cumsum(child_count)
    return SidTrie(items=items, node_ptr=node_ptr.astype(np.int32),
                   edge_tok=np.concatenate(edge_tok).astype(np.int32),
                   edge_child=np.concatenate(edge_child).astype(np.int32),
                   level_start=level_start.astype(np.int32), V=V)


@dataclasses.dataclass
class TrieSelectInputs:
    """One constrained selection call: a SelectInputs batch whose beams each
    hold a semantic-ID prefix of `step` tokens taken from the catalog, the
    trie node of that prefix, and the trie."""

    sel: SelectInputs
    trie: SidTrie
    sid: np.ndarray        # [R_old][step] i32, each beam's prefix tokens
    node_old: np.ndarray   # [R_old] i32, trie node of the prefix (-1: none)
    step: int


def trie_select_inputs(W_old: Sequence[int], W_new: Sequence[int], V: int, step: int,
                       trie: SidTrie, seed: int, dead: float = 0.0,
                       logit_std: float = 2.0, score_spread: float = 3.0) -> TrieSelectInputs:
    """Beams whose prefixes are the first `step` tokens of random catalog
    items (a fraction `dead` get a prefix no item has, node -1); scores and
    logits as select_inputs."""
    sel = select_inputs(W_old, W_new, V, seed, logit_std=logit_std, score_spread=score_spread)
    rng = np.random.default_rng(seed + 7919)
    R = int(sel.row_offset_old[-1])
    pick = rng.integers(0, trie.items.shape[0], size=R)
    sid = trie.items[pick, :step].astype(np.int32).reshape(R, step)
    node = trie.node_of(sid) if R else np.zeros(0, np.int32)
    if dead > 0 and step > 0 and R:
        kill = rng.random(R) < dead
        for r in np.nonzero(kill)[0]:
            for _ in range(64):
                cand = rng.integers(0, V, size=step).astype(np.int32)
                if trie.node_of(cand[None, :])[0] < 0:
                    sid[r] = cand
                    node[r] = -1
                    break
    return TrieSelectInputs(sel=sel, trie=trie, sid=sid, node_old=node.astype(np.int32), step=step)


# Constrained selection at the 900-beam shape: a synthetic catalog of one
# million 3-token items over the 8192-token vocabulary; the benchmarked call
# is the second step (each beam holds one token; ~120 legal next tokens).
TRIE_CATALOG = dict(n_items=1_000_000, depth=3, V=8192, seed=9001)
TRIE_WORKLOADS = {
    4: dict(name="w900_b4_v8192_items1m_step1", W_old=(900,) * 4, W_new=(900,) * 4, step=1,
            seed=4507),
}

_trie_cache: Dict[tuple, SidTrie] = {}


def catalog_trie(n_items: int, depth: int, V: int, seed: int) -> SidTrie:
    key = (n_items, depth, V, seed)
    if key not in _trie_cache:
        _trie_cache[key] = build_trie(sid_catalog(n_items, depth, V, seed), V)
    return _trie_cache[key]


def trie_workload(cfg: int) -> TrieSelectInputs:
    w = dict(TRIE_WORKLOADS[cfg])
    w.pop("name")
    trie = catalog_trie(**TRIE_CATALOG)
    return trie_select_inputs(trie=trie, V=TRIE_CATALOG["V"], **w)
