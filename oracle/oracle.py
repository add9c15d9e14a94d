"""The oracle: plain, slow, fp64 CPU definitions of what the device path
computes.  Test infrastructure only (tests, the smoke check and the CPU
baseline of the benchmark use it; the library never does).

Decode attention and the beam step are written in C (``oracle.c``, which
states the definitions); this module compiles that with gcc and marshals
numpy buffers for them.  Beam selection, the paged-context gather and the
trie-constrained selection are written here in numpy, each citing the
passage it follows.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    global _lib
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def default_threads() -> int:
    """Host threads for the oracle: every CPU this process may run on, or
    fewer when OMP_NUM_THREADS allots fewer (a machine's share for one job)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _open(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int, ctypes.c_int64
    lib.oracle_decode_attn.argtypes = [i32, i32, i32, i32, i32, i32, i64, i64,
                                       ctypes.c_double, P, P, P, P, P, P, P, P, P,
                                       P, i32, P, P, i32]
    lib.oracle_decode_attn.restype = i32
    lib.oracle_beam_step.argtypes = [i32, i32, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P,
                                     P, P]
    lib.oracle_beam_step.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _open(_LIB)
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode_attn(q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len,
                row_offset, scale: Optional[float] = None,
                rows: Optional[Sequence[int]] = None, n_threads: Optional[int] = None):
    """fp64 attention of each packed row over its request's context ++ its BeamPath tokens.

    bf16 tensors are uint16 bit arrays in the library's layouts:
    q [R][Hq][D], ctx_k/ctx_v [B][ctx_cap][Hkv][D], beam_k/beam_v
    [B][beam_cap][Hkv][D]; beam_path [R][T_cap] int32; ctx_len, beam_len [B],
    row_offset [B+1] int32.  Returns (out [n][Hq][D] float64, lse [n][Hq]
    float64) for ``rows`` (all R rows by default), lse in natural log.
    """
    return _call(_load(), q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len,
                 row_offset, scale, rows, n_threads)


def from_library(path: str):
    """``decode_attn`` bound to another build of oracle.c (the tests compile
    deliberately broken copies to show that the pins reject them)."""
    lib = _open(path)

    def fn(q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len, row_offset,
           scale=None, rows=None, n_threads=None):
        return _call(lib, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len,
                     row_offset, scale, rows, n_threads)
    return fn


def _call(lib, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len, row_offset,
          scale, rows, n_threads):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    ctx_k = np.ascontiguousarray(ctx_k, dtype=np.uint16)
    ctx_v = np.ascontiguousarray(ctx_v, dtype=np.uint16)
    beam_k = np.ascontiguousarray(beam_k, dtype=np.uint16)
    beam_v = np.ascontiguousarray(beam_v, dtype=np.uint16)
    ctx_len = np.ascontiguousarray(ctx_len, dtype=np.int32)
    beam_len = np.ascontiguousarray(beam_len, dtype=np.int32)
    row_offset = np.ascontiguousarray(row_offset, dtype=np.int32)
    beam_path = np.ascontiguousarray(beam_path, dtype=np.int32)
    R, Hq, D = q.shape
    B, ctx_cap, Hkv, D2 = ctx_k.shape
    assert D2 == D and beam_k.shape[0] == B and beam_k.shape[2:] == (Hkv, D)
    assert ctx_v.shape == ctx_k.shape and beam_v.shape == beam_k.shape
    assert beam_path.ndim == 2 and beam_path.shape[0] == R
    T_cap = beam_path.shape[1]
    beam_cap = beam_k.shape[1]
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n = R if rows_arr is None else int(rows_arr.size)
    out = np.zeros((n, Hq, D), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    if n_threads is None:
        n_threads = default_threads()
    st = lib.oracle_decode_attn(B, R, Hq, Hkv, D, T_cap, ctx_cap, beam_cap, float(scale),
                                _ptr(q), _ptr(ctx_k), _ptr(ctx_v), _ptr(ctx_len), _ptr(beam_k),
                                _ptr(beam_v), _ptr(beam_path), _ptr(beam_len), _ptr(row_offset),
                                _ptr(rows_arr), n, _ptr(out), _ptr(lse), int(n_threads))
    if st != 0:
        raise RuntimeError(f"oracle_decode_attn failed with status {st}")
    return out, lse


def decode_attn_inputs(inp, rows=None, n_threads=None):
    """Run the oracle on a generated ``Inputs`` object."""
    return decode_attn(inp.q, inp.ctx_k, inp.ctx_v, inp.ctx_len, inp.beam_k, inp.beam_v,
                       inp.beam_path, inp.beam_len, inp.row_offset, scale=inp.scale,
                       rows=rows, n_threads=n_threads)


def beam_step(row_offset_old, row_offset_new, parent, path_old, beam_len_old, new_k, new_v,
              path_new, beam_k, beam_v, W_cap: int, lib=None):
    """BeamKV append + BeamPath update of one decode step (see ``oracle_beam_step``).

    ``path_new`` [R_new][T_cap] int32, ``beam_k``/``beam_v`` [B][beam_cap][Hkv][D]
    uint16 are the state before the step; copies are updated and returned as
    (path_new, beam_len_new, beam_k, beam_v, n_skipped_rows).
    """
    lib = _load() if lib is None else lib
    row_offset_old = np.ascontiguousarray(row_offset_old, dtype=np.int32)
    row_offset_new = np.ascontiguousarray(row_offset_new, dtype=np.int32)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    path_old = np.ascontiguousarray(path_old, dtype=np.int32)
    beam_len_old = np.ascontiguousarray(beam_len_old, dtype=np.int32)
    new_k = np.ascontiguousarray(new_k, dtype=np.uint16)
    new_v = np.ascontiguousarray(new_v, dtype=np.uint16)
    path_new = np.array(path_new, dtype=np.int32, copy=True)
    beam_k = np.array(beam_k, dtype=np.uint16, copy=True)
    beam_v = np.array(beam_v, dtype=np.uint16, copy=True)
    B = row_offset_new.size - 1
    assert row_offset_old.size == B + 1 and beam_len_old.size == B
    B2, beam_cap, Hkv, D = beam_k.shape
    assert B2 == B and beam_v.shape == beam_k.shape
    R_new = int(row_offset_new[-1])
    T_cap = path_new.shape[1]
    assert path_new.shape[0] == R_new and parent.size >= R_new
    assert path_old.ndim == 2 and path_old.shape[1] == T_cap
    assert new_k.shape == (R_new, Hkv, D) and new_v.shape == new_k.shape
    len_new = np.zeros(B, dtype=np.int32)
    st = lib.oracle_beam_step(B, Hkv, D, T_cap, int(W_cap), beam_cap, _ptr(row_offset_old),
                              _ptr(row_offset_new), _ptr(parent), _ptr(path_old),
                              _ptr(beam_len_old), _ptr(new_k), _ptr(new_v), _ptr(path_new),
                              _ptr(len_new), _ptr(beam_k), _ptr(beam_v))
    if st < 0:
        raise RuntimeError(f"oracle_beam_step failed with status {st}")
    return path_new, len_new, beam_k, beam_v, int(st)


def beam_step_from_library(path: str):
    """``beam_step`` bound to another build of oracle.c (broken copies in tests)."""
    lib = _open(path)

    def fn(*args, **kw):
        return beam_step(*args, lib=lib, **kw)
    return fn


def gather_pages(k_pages, v_pages, page_table, page_size: int, ctx_len, ctx_cap: int):
    """Dense ContextKV [B][ctx_cap][Hkv][D] from pages: token j < ctx_len[b] of
    request b is row j % page_size of page page_table[b][j // page_size]
    (tokens past ctx_len are NaN).  A plain loop over tokens; the page
    layout is the only thing it adds to the dense definition."""
    page_table = np.asarray(page_table)
    B = page_table.shape[0]
    _, ps, Hkv, D = k_pages.shape
    assert ps == page_size
    k = np.full((B, ctx_cap, Hkv, D), 0x7FC0, dtype=np.uint16)
    v = np.full((B, ctx_cap, Hkv, D), 0x7FC0, dtype=np.uint16)
    for b in range(B):
        for j in range(int(ctx_len[b])):
            page = int(page_table[b, j // page_size])
            k[b, j] = k_pages[page, j % page_size]
            v[b, j] = v_pages[page, j % page_size]
    return k, v


def decode_attn_paged(q, k_pages, v_pages, page_table, page_size, ctx_len, beam_k, beam_v,
                      beam_path, beam_len, row_offset, ctx_cap=None, scale=None, rows=None,
                      n_threads=None):
    """``decode_attn`` over a paged ContextKV (gathered to dense first)."""
    if ctx_cap is None:
        ctx_cap = max(int(np.max(ctx_len, initial=0)), 1)
    k, v = gather_pages(k_pages, v_pages, page_table, page_size, ctx_len, ctx_cap)
    return decode_attn(q, k, v, ctx_len, beam_k, beam_v, beam_path, beam_len, row_offset,
                       scale=scale, rows=rows, n_threads=n_threads)


def beam_select(row_offset_old, row_offset_new, score_old, logits):
    """Beam selection of one decode step, in fp64 (xGR review, section "xBeam";
    SID-GR README, "Roadmap": log_softmax + top-K + beam selection).

    Request b's candidates are (w, v) over its old beams w and the vocabulary
    v, with value score_old[w] + log_softmax(logits[w])[v] (natural log).  The
    K_b = row_offset_new[b+1] - row_offset_new[b] best are kept, ordered by
    value (larger first) and, among equal values, by the flat index w*V + v
    (smaller first).  Returns (score_new [R_new], parent [R_new] (w within
    the request), token [R_new]) packed like row_offset_new; a request with
    fewer candidates than K_b fills the rest with (-inf, -1, -1).
    """
    row_offset_old = np.asarray(row_offset_old)
    row_offset_new = np.asarray(row_offset_new)
    logits = np.asarray(logits, dtype=np.float64)
    score_old = np.asarray(score_old, dtype=np.float64)
    B = row_offset_new.size - 1
    V = logits.shape[1] if logits.ndim == 2 else 0
    R_new = int(row_offset_new[-1])
    score_new = np.full(R_new, -np.inf)
    parent = np.full(R_new, -1, dtype=np.int32)
    token = np.full(R_new, -1, dtype=np.int32)
    for b in range(B):
        r0, r1 = int(row_offset_old[b]), int(row_offset_old[b + 1])
        k0, k1 = int(row_offset_new[b]), int(row_offset_new[b + 1])
        if r1 == r0 or V == 0:
            continue
        x = logits[r0:r1]                                        # [W][V]
        m = x.max(axis=1, keepdims=True)
        lse = m + np.log(np.exp(x - m).sum(axis=1, keepdims=True))
        value = (score_old[r0:r1, None] + x - lse).ravel()       # flat index w*V + v
        flat = np.arange(value.size)
        order = np.lexsort((flat, -value))                       # value desc, then index asc
        n = min(k1 - k0, value.size)
        sel = order[:n]
        score_new[k0:k0 + n] = value[sel]
        parent[k0:k0 + n] = sel // V
        token[k0:k0 + n] = sel % V
    return score_new, parent, token


def trie_walk(node_ptr, edge_tok, edge_child, prefix) -> int:
    """Node reached from the root by following `prefix` token by token in a
    CSR trie (node u's children: edges node_ptr[u] .. node_ptr[u+1]-1, edge e
    labelled edge_tok[e], leading to edge_child[e]); -1 once a token has no
    edge (GR-Inference blog, kernel design: prefix traversal of the SID trie).
    Each level scans all of the node's edges."""
    node = 0
    for t in prefix:
        lo, hi = int(node_ptr[node]), int(node_ptr[node + 1])
        hit = np.nonzero(np.asarray(edge_tok[lo:hi]) == int(t))[0]
        if hit.size == 0:
            return -1
        node = int(edge_child[lo + int(hit[0])])
    return node


def beam_select_trie(row_offset_old, row_offset_new, score_old, logits, sid, node_ptr,
                     edge_tok, edge_child):
    """Item-constrained beam selection of one decode step, in fp64
    (GR-Inference blog, kernel design: the item-constrained kernel does
    prefix traversal, legal-token gather and local top-K over the SID trie;
    xGR review, section "xBeam").

    Beam w of request b holds the token prefix sid[w]; its legal next tokens
    are the labels of the edges leaving the node that prefix reaches (none if
    the prefix leaves the trie).  Candidate (w, t), t legal, is valued
    score_old[w] + logits[w][t] - ln sum_{legal u} exp(logits[w][u]): the
    log-softmax over the legal tokens only, i.e. with every other logit masked
    to -inf.  Ranking, packing and padding as beam_select.  Returns
    (score_new, parent, token, node_new), node_new the node of the kept
    beam's extended prefix (-1 for padding).
    """
    row_offset_old = np.asarray(row_offset_old)
    row_offset_new = np.asarray(row_offset_new)
    logits = np.asarray(logits, dtype=np.float64)
    score_old = np.asarray(score_old, dtype=np.float64)
    B = row_offset_new.size - 1
    V = logits.shape[1] if logits.ndim == 2 else 0
    R_new = int(row_offset_new[-1])
    score_new = np.full(R_new, -np.inf)
    parent = np.full(R_new, -1, dtype=np.int32)
    token = np.full(R_new, -1, dtype=np.int32)
    node_new = np.full(R_new, -1, dtype=np.int32)
    for b in range(B):
        r0, r1 = int(row_offset_old[b]), int(row_offset_old[b + 1])
        k0, k1 = int(row_offset_new[b]), int(row_offset_new[b + 1])
        vals, flats, kids = [], [], []
        for w in range(r1 - r0):
            node = trie_walk(node_ptr, edge_tok, edge_child, sid[r0 + w])
            if node < 0:
                continue
            lo, hi = int(node_ptr[node]), int(node_ptr[node + 1])
            if hi == lo:
                continue
            legal = np.asarray(edge_tok[lo:hi], dtype=np.int64)
            x = logits[r0 + w, legal]
            m = x.max()
            lse = m + np.log(np.exp(x - m).sum())
            vals.append(score_old[r0 + w] + x - lse)
            flats.append(w * V + legal)
            kids.append(np.asarray(edge_child[lo:hi]))
        if not vals:
            continue
        value = np.concatenate(vals)
        flat = np.concatenate(flats)
        kid = np.concatenate(kids)
        order = np.lexsort((flat, -value))                       # value desc, then index asc
        n = min(k1 - k0, value.size)
        sel = order[:n]
        score_new[k0:k0 + n] = value[sel]
        parent[k0:k0 + n] = flat[sel] // V
        token[k0:k0 + n] = flat[sel] % V
        node_new[k0:k0 + n] = kid[sel]
    return score_new, parent, token, node_new
