"""Python binding of the C ABI in include/gr_attn.h (ctypes).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in libgr_attn.so.
Loading fails loudly when the library has not been built.

Functions with the C names take the same arguments as the C entry points
(a dims struct plus raw pointers); ``decode_attn`` / ``decode_attn_generic``
/ ``check_metadata`` / ``beam_step`` accept torch tensors.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgr_attn.so")

GR_OK = 0
GR_ERR_NULL = -1
GR_ERR_DIMS = -2
GR_ERR_UNSUPPORTED = -3
GR_ERR_ALIGN = -4
GR_ERR_LAUNCH = -5
GR_ERR_DEVICE = -6
GR_ERR_WORKSPACE = -7
GR_FLAG_TILING = 0x40000000
GR_FLAG_ROW16 = 0x20000000


def tiling_flags(tiling) -> int:
    """dims flags for a forced (nqt, nks[, n_split[, row16]]) work
    decomposition (GR_TILING / GR_TILING16 in include/gr_attn.h); row16
    selects waves of 16 stacked rows.  None -> 0 (the library plans)."""
    if tiling is None:
        return 0
    nqt, nks, *rest = tiling
    split = rest[0] if rest else 1
    row16 = bool(rest[1]) if len(rest) > 1 else False
    return GR_FLAG_TILING | (GR_FLAG_ROW16 if row16 else 0) | int(nqt) | (int(nks) << 8) | \
        (int(split) << 16)

EXPORTS = ("gr_decode_attn_workspace_bytes", "gr_decode_attn_plan", "gr_decode_attn",
           "gr_decode_attn_noalloc",
           "gr_decode_attn_generic", "gr_decode_attn_paged",
           "gr_check_metadata", "gr_beam_step", "gr_beam_select_workspace_bytes",
           "gr_beam_select", "gr_beam_select_trie", "gr_status_str", "gr_version")


class Dims(ctypes.Structure):
    """``gr_decode_attn_dims`` (host memory)."""

    _fields_ = [("B", ctypes.c_int32), ("R", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("W_max", ctypes.c_int32),
                ("T_cap", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("ctx_cap", ctypes.c_int64), ("beam_cap", ctypes.c_int64),
                ("scale", ctypes.c_float), ("flags", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64)]


class StepDims(ctypes.Structure):
    """``gr_beam_step_dims`` (host memory)."""

    _fields_ = [("B", ctypes.c_int32), ("R_old", ctypes.c_int32), ("R_new", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("T_cap", ctypes.c_int32),
                ("W_cap", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("beam_cap", ctypes.c_int64)]


class SelectDims(ctypes.Structure):
    """``gr_beam_select_dims`` (host memory)."""

    _fields_ = [("B", ctypes.c_int32), ("R_old", ctypes.c_int32), ("R_new", ctypes.c_int32),
                ("V", ctypes.c_int32), ("K_max", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SidTrie(ctypes.Structure):
    """``gr_sid_trie`` (host memory holding device pointers)."""

    _fields_ = [("node_ptr", ctypes.c_void_p), ("edge_tok", ctypes.c_void_p),
                ("edge_child", ctypes.c_void_p), ("n_nodes", ctypes.c_int32),
                ("n_edges", ctypes.c_int32), ("max_fanout", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class PagedCtx(ctypes.Structure):
    """``gr_paged_ctx`` (host memory holding device pointers)."""

    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("pages_per_req", ctypes.c_int32), ("n_pages", ctypes.c_int64)]


class GrAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({gr_status_str(status)})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libgr_attn.so; raise if it is missing (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m shared_prefix_beam_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        DP = ctypes.POINTER(Dims)
        attn_args = [DP, P, P, P, P, P, P, P, P, P, P, P, P]
        for name in ("gr_decode_attn", "gr_decode_attn_noalloc", "gr_decode_attn_generic"):
            fn = getattr(lib, name)
            fn.argtypes = attn_args
            fn.restype = ctypes.c_int
        lib.gr_decode_attn_workspace_bytes.argtypes = [DP]
        lib.gr_decode_attn_workspace_bytes.restype = ctypes.c_size_t
        lib.gr_decode_attn_plan.argtypes = [DP, ctypes.POINTER(ctypes.c_int32)]
        lib.gr_decode_attn_plan.restype = ctypes.c_int
        lib.gr_check_metadata.argtypes = [DP, P, P, P, P, P, P]
        lib.gr_check_metadata.restype = ctypes.c_int
        lib.gr_decode_attn_paged.argtypes = [DP, ctypes.POINTER(PagedCtx)] + [P] * 10
        lib.gr_decode_attn_paged.restype = ctypes.c_int
        lib.gr_beam_step.argtypes = [ctypes.POINTER(StepDims)] + [P] * 13
        lib.gr_beam_step.restype = ctypes.c_int
        SDP = ctypes.POINTER(SelectDims)
        lib.gr_beam_select_workspace_bytes.argtypes = [SDP]
        lib.gr_beam_select_workspace_bytes.restype = ctypes.c_size_t
        lib.gr_beam_select.argtypes = [SDP] + [P] * 8 + [ctypes.c_size_t, P]
        lib.gr_beam_select.restype = ctypes.c_int
        lib.gr_beam_select_trie.argtypes = [SDP, ctypes.POINTER(SidTrie)] + [P] * 9 + \
            [P, ctypes.c_size_t, P]
        lib.gr_beam_select_trie.restype = ctypes.c_int
        lib.gr_status_str.argtypes = [ctypes.c_int]
        lib.gr_status_str.restype = ctypes.c_char_p
        lib.gr_version.argtypes = []
        lib.gr_version.restype = ctypes.c_int
        _lib = lib
    return _lib


# ---- the C entry points, same names and arguments -------------------------
def gr_decode_attn_workspace_bytes(dims: Dims) -> int:
    return load().gr_decode_attn_workspace_bytes(ctypes.byref(dims))


def gr_decode_attn(dims: Dims, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v,
                   beam_path, beam_len, out, lse, stream) -> int:
    return load().gr_decode_attn(ctypes.byref(dims), row_offset, q, ctx_k, ctx_v, ctx_len,
                                 beam_k, beam_v, beam_path, beam_len, out, lse, stream)


def gr_decode_attn_noalloc(dims: Dims, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v,
                           beam_path, beam_len, out, lse, stream) -> int:
    return load().gr_decode_attn_noalloc(ctypes.byref(dims), row_offset, q, ctx_k, ctx_v,
                                         ctx_len, beam_k, beam_v, beam_path, beam_len, out,
                                         lse, stream)


def gr_decode_attn_generic(dims: Dims, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v,
                           beam_path, beam_len, out, lse, stream) -> int:
    return load().gr_decode_attn_generic(ctypes.byref(dims), row_offset, q, ctx_k, ctx_v,
                                         ctx_len, beam_k, beam_v, beam_path, beam_len, out,
                                         lse, stream)


def gr_decode_attn_paged(dims: Dims, ctx: PagedCtx, row_offset, q, ctx_len, beam_k, beam_v,
                         beam_path, beam_len, out, lse, stream) -> int:
    return load().gr_decode_attn_paged(ctypes.byref(dims), ctypes.byref(ctx), row_offset, q,
                                       ctx_len, beam_k, beam_v, beam_path, beam_len, out, lse,
                                       stream)


def gr_check_metadata(dims: Dims, row_offset, ctx_len, beam_path, beam_len, violations,
                      stream) -> int:
    return load().gr_check_metadata(ctypes.byref(dims), row_offset, ctx_len, beam_path,
                                    beam_len, violations, stream)


def gr_beam_step(dims: StepDims, row_offset_old, row_offset_new, parent, path_old,
                 beam_len_old, new_k, new_v, path_new, beam_len_new, beam_k, beam_v, violations,
                 stream) -> int:
    return load().gr_beam_step(ctypes.byref(dims), row_offset_old, row_offset_new, parent,
                               path_old, beam_len_old, new_k, new_v, path_new, beam_len_new,
                               beam_k, beam_v, violations, stream)


def gr_beam_select_workspace_bytes(dims: SelectDims) -> int:
    return load().gr_beam_select_workspace_bytes(ctypes.byref(dims))


def gr_beam_select(dims: SelectDims, row_offset_old, row_offset_new, score_old, logits,
                   score_new, parent, token, workspace, workspace_bytes: int, stream) -> int:
    return load().gr_beam_select(ctypes.byref(dims), row_offset_old, row_offset_new, score_old,
                                 logits, score_new, parent, token, workspace,
                                 int(workspace_bytes), stream)


def gr_beam_select_trie(dims: SelectDims, trie: SidTrie, row_offset_old, row_offset_new,
                        score_old, logits, node_old, score_new, parent, token, node_new,
                        workspace, workspace_bytes: int, stream) -> int:
    return load().gr_beam_select_trie(ctypes.byref(dims), ctypes.byref(trie), row_offset_old,
                                      row_offset_new, score_old, logits, node_old, score_new,
                                      parent, token, node_new, workspace, int(workspace_bytes),
                                      stream)


def gr_status_str(status: int) -> str:
    return load().gr_status_str(int(status)).decode()


def gr_version() -> int:
    return load().gr_version()


# ---- torch front end -------------------------------------------------------
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def make_dims(q, ctx_k, beam_k, beam_path, W_max: int, scale: Optional[float] = None,
              tiling=None) -> Dims:
    R, Hq, D = q.shape
    B, ctx_cap, Hkv, _ = ctx_k.shape
    return Dims(B=B, R=R, Hq=Hq, Hkv=Hkv, D=D, W_max=int(W_max), T_cap=beam_path.shape[1],
                reserved=0, ctx_cap=ctx_cap, beam_cap=beam_k.shape[1],
                scale=0.0 if scale is None else float(scale), flags=tiling_flags(tiling))


def plan(dims: Dims) -> dict:
    """The work decomposition the library plans for ``dims``
    (gr_decode_attn_plan): nqt, nks, n_split, row16, grid."""
    out = (ctypes.c_int32 * 5)()
    st = load().gr_decode_attn_plan(ctypes.byref(dims), out)
    if st != GR_OK:
        raise GrAttnError(st, "gr_decode_attn_plan")
    return dict(nqt=out[0], nks=out[1], n_split=out[2], row16=bool(out[3]), grid=out[4])


def attach_workspace(dims: Dims, workspace, device):
    """Point ``dims`` at a workspace of gr_decode_attn_workspace_bytes(dims)
    bytes: ``workspace`` (a device tensor, zero-filled before its first use)
    or, when None, a fresh zero-filled uint8 tensor.  Returns the tensor (or
    None when the call needs no workspace); keep it alive until the call has
    run."""
    import torch
    need = gr_decode_attn_workspace_bytes(dims)
    if need == 0:
        dims.workspace, dims.workspace_bytes = None, 0
        return workspace
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=device)
    dims.workspace = workspace.data_ptr()
    dims.workspace_bytes = workspace.numel() * workspace.element_size()
    return workspace


def _check(q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len, row_offset):
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("ctx_k", ctx_k, torch.bfloat16),
                        ("ctx_v", ctx_v, torch.bfloat16), ("beam_k", beam_k, torch.bfloat16),
                        ("beam_v", beam_v, torch.bfloat16), ("ctx_len", ctx_len, torch.int32),
                        ("beam_len", beam_len, torch.int32),
                        ("beam_path", beam_path, torch.int32),
                        ("row_offset", row_offset, torch.int32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 3 or ctx_k.dim() != 4 or beam_k.dim() != 4 or beam_path.dim() != 2:
        raise ValueError("bad tensor ranks")
    if ctx_v.shape != ctx_k.shape or beam_v.shape != beam_k.shape:
        raise ValueError("K and V shapes differ")
    B = ctx_k.shape[0]
    if beam_k.shape[0] != B or ctx_len.numel() != B or beam_len.numel() != B \
            or row_offset.numel() != B + 1 or beam_path.shape[0] != q.shape[0]:
        raise ValueError("request count mismatch")
    if ctx_k.shape[2:] != beam_k.shape[2:] or ctx_k.shape[3] != q.shape[2]:
        raise ValueError("head layout mismatch")


def _run(fn_name, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len, row_offset,
         W_max, scale, out, lse, stream, workspace=None, tiling=None) -> Tuple:
    import torch
    _check(q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len, row_offset)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    dims = make_dims(q, ctx_k, beam_k, beam_path, W_max, scale,
                     tiling if fn_name == "fused" else None)
    if fn_name == "fused":
        workspace = attach_workspace(dims, workspace, q.device)
    fn = gr_decode_attn if fn_name == "fused" else gr_decode_attn_generic
    st = fn(dims, _ptr(row_offset), _ptr(q), _ptr(ctx_k), _ptr(ctx_v), _ptr(ctx_len),
            _ptr(beam_k), _ptr(beam_v), _ptr(beam_path), _ptr(beam_len), _ptr(out), _ptr(lse),
            _stream_handle(stream))
    if st != GR_OK:
        raise GrAttnError(st, "gr_decode_attn" if fn_name == "fused" else
                          "gr_decode_attn_generic")
    return out, lse


def decode_attn(q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len, row_offset,
                W_max: int, scale: Optional[float] = None, out=None, lse=None, stream=None,
                workspace=None, tiling=None):
    """Fused shared-context / BeamPath / LSE-merge decode attention.

    Tensors as in include/gr_attn.h (bf16 / int32, contiguous, on the GPU).
    ``W_max`` bounds every request's row count.  ``workspace``: a device
    tensor of at least gr_decode_attn_workspace_bytes bytes, zero-filled
    before its first use and not shared by concurrent calls (None: a fresh
    one per call).  ``tiling``: (nqt, nks[, n_split]) forces the work
    decomposition (tuning and tests); None lets the library plan.  Returns
    (out bf16 [R,Hq,D], lse fp32 [R,Hq]); enqueued on ``stream`` (default:
    torch's current one).
    """
    return _run("fused", q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len,
                row_offset, W_max, scale, out, lse, stream, workspace, tiling)


def decode_attn_generic(q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len,
                        row_offset, W_max: int, scale: Optional[float] = None, out=None,
                        lse=None, stream=None):
    """Same result through the generic per-row comparator kernel."""
    return _run("generic", q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path, beam_len,
                row_offset, W_max, scale, out, lse, stream)


def decode_attn_paged(q, k_pages, v_pages, page_table, page_size: int, ctx_len, beam_k, beam_v,
                      beam_path, beam_len, row_offset, W_max: int, ctx_cap: Optional[int] = None,
                      scale: Optional[float] = None, out=None, lse=None, stream=None,
                      workspace=None, tiling=None):
    """``decode_attn`` with the ContextKV in pages (include/gr_attn.h,
    gr_decode_attn_paged): k_pages / v_pages bf16 [n_pages][page_size][Hkv][D],
    page_table int32 [B][pages_per_req].  ``ctx_cap`` defaults to
    pages_per_req * page_size."""
    import torch
    n_pages, ps, Hkv, D = k_pages.shape
    if ps != page_size or v_pages.shape != k_pages.shape:
        raise ValueError("page pool shape mismatch")
    if page_table.dtype != torch.int32 or not page_table.is_cuda or page_table.dim() != 2 \
            or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous int32 [B][pages_per_req] device tensor")
    B, ppr = page_table.shape
    cap = ppr * page_size if ctx_cap is None else int(ctx_cap)
    for name, t, dt in (("q", q, torch.bfloat16), ("k_pages", k_pages, torch.bfloat16),
                        ("v_pages", v_pages, torch.bfloat16), ("ctx_len", ctx_len, torch.int32),
                        ("beam_k", beam_k, torch.bfloat16), ("beam_v", beam_v, torch.bfloat16),
                        ("beam_path", beam_path, torch.int32), ("beam_len", beam_len, torch.int32),
                        ("row_offset", row_offset, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    if beam_k.shape[0] != B or ctx_len.numel() != B or beam_len.numel() != B \
            or row_offset.numel() != B + 1 or beam_path.shape[0] != q.shape[0] \
            or beam_k.shape[2:] != (Hkv, D) or q.shape[2] != D:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    R, Hq, _ = q.shape
    dims = Dims(B=B, R=R, Hq=Hq, Hkv=Hkv, D=D, W_max=int(W_max), T_cap=beam_path.shape[1],
                reserved=0, ctx_cap=cap, beam_cap=beam_k.shape[1],
                scale=0.0 if scale is None else float(scale), flags=tiling_flags(tiling))
    workspace = attach_workspace(dims, workspace, q.device)
    ctx = PagedCtx(k_pages=k_pages.data_ptr(), v_pages=v_pages.data_ptr(),
                   page_table=page_table.data_ptr(), page_size=int(page_size), pages_per_req=ppr,
                   n_pages=n_pages)
    st = gr_decode_attn_paged(dims, ctx, _ptr(row_offset), _ptr(q), _ptr(ctx_len), _ptr(beam_k),
                              _ptr(beam_v), _ptr(beam_path), _ptr(beam_len), _ptr(out),
                              _ptr(lse), _stream_handle(stream))
    if st != GR_OK:
        raise GrAttnError(st, "gr_decode_attn_paged")
    return out, lse


def check_metadata(ctx_len, beam_path, beam_len, row_offset, *, B, R, Hq, Hkv, D, W_max,
                   ctx_cap, beam_cap, violations=None, stream=None):
    """Device-side precondition check; returns the int32 violation count tensor."""
    import torch
    if violations is None:
        violations = torch.zeros(1, dtype=torch.int32, device=row_offset.device)
    dims = Dims(B=B, R=R, Hq=Hq, Hkv=Hkv, D=D, W_max=W_max, T_cap=beam_path.shape[1],
                reserved=0, ctx_cap=ctx_cap, beam_cap=beam_cap, scale=0.0, flags=0)
    st = gr_check_metadata(dims, _ptr(row_offset), _ptr(ctx_len), _ptr(beam_path),
                           _ptr(beam_len), _ptr(violations), _stream_handle(stream))
    if st != GR_OK:
        raise GrAttnError(st, "gr_check_metadata")
    return violations


def beam_step(row_offset_old, row_offset_new, parent, path_old, beam_len_old, new_k, new_v,
              path_new, beam_len_new, beam_k, beam_v, W_cap: int, violations=None,
              stream=None):
    """BeamKV append + BeamPath update of one decode step (include/gr_attn.h).

    Writes ``path_new``, ``beam_len_new`` and the new slots of ``beam_k`` /
    ``beam_v`` in place; enqueued on ``stream`` (default: torch's current
    one).  ``violations`` (int32 [1] on the device, or None) accumulates the
    rows skipped as out of range.
    """
    import torch
    for name, t, dt in (("row_offset_old", row_offset_old, torch.int32),
                        ("row_offset_new", row_offset_new, torch.int32),
                        ("parent", parent, torch.int32), ("path_old", path_old, torch.int32),
                        ("beam_len_old", beam_len_old, torch.int32),
                        ("new_k", new_k, torch.bfloat16), ("new_v", new_v, torch.bfloat16),
                        ("path_new", path_new, torch.int32),
                        ("beam_len_new", beam_len_new, torch.int32),
                        ("beam_k", beam_k, torch.bfloat16), ("beam_v", beam_v, torch.bfloat16)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    B, beam_cap, Hkv, D = beam_k.shape
    if beam_v.shape != beam_k.shape or new_v.shape != new_k.shape:
        raise ValueError("K and V shapes differ")
    R_new = new_k.shape[0]
    if new_k.shape[1:] != (Hkv, D) or path_new.shape[0] != R_new or parent.numel() < R_new:
        raise ValueError("new-row shapes mismatch")
    if row_offset_old.numel() != B + 1 or row_offset_new.numel() != B + 1 \
            or beam_len_old.numel() != B or beam_len_new.numel() != B:
        raise ValueError("request count mismatch")
    if path_old.dim() != 2 or path_old.shape[1] != path_new.shape[1]:
        raise ValueError("BeamPath tables must share T_cap")
    dims = StepDims(B=B, R_old=path_old.shape[0], R_new=R_new, Hkv=Hkv, D=D,
                    T_cap=path_new.shape[1], W_cap=int(W_cap), reserved=0, beam_cap=beam_cap)
    st = gr_beam_step(dims, _ptr(row_offset_old), _ptr(row_offset_new), _ptr(parent),
                      _ptr(path_old), _ptr(beam_len_old), _ptr(new_k), _ptr(new_v),
                      _ptr(path_new), _ptr(beam_len_new), _ptr(beam_k), _ptr(beam_v),
                      _ptr(violations), _stream_handle(stream))
    if st != GR_OK:
        raise GrAttnError(st, "gr_beam_step")


def beam_select(row_offset_old, row_offset_new, score_old, logits, K_max: int, *, R_new=None,
                score_new=None, parent=None, token=None, workspace=None, stream=None):
    """log_softmax + top-K beam selection of one decode step (include/gr_attn.h).

    ``row_offset_new`` gives every request's kept-beam count; ``K_max`` bounds
    it and ``R_new`` (= row_offset_new[-1]) sizes the outputs when they are
    not passed.  Returns (score_new fp32, parent int32, token int32) of
    length R_new, enqueued on ``stream`` (default: torch's current one).
    """
    import torch
    for name, t, dt in (("row_offset_old", row_offset_old, torch.int32),
                        ("row_offset_new", row_offset_new, torch.int32),
                        ("score_old", score_old, torch.float32),
                        ("logits", logits, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if logits.dim() != 2:
        raise ValueError("logits must be [R_old, V]")
    R_old, V = logits.shape
    B = row_offset_old.numel() - 1
    if row_offset_new.numel() != B + 1 or score_old.numel() != R_old:
        raise ValueError("request or row count mismatch")
    if R_new is None:
        if score_new is None:
            raise ValueError("pass R_new or the output tensors")
        R_new = score_new.numel()
    dev = logits.device
    if score_new is None:
        score_new = torch.empty(R_new, dtype=torch.float32, device=dev)
    if parent is None:
        parent = torch.empty(R_new, dtype=torch.int32, device=dev)
    if token is None:
        token = torch.empty(R_new, dtype=torch.int32, device=dev)
    for name, t, dt in (("score_new", score_new, torch.float32), ("parent", parent, torch.int32),
                        ("token", token, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous() or t.numel() != R_new:
            raise ValueError(f"{name} must be a contiguous device {dt} tensor of {R_new}")
    dims = SelectDims(B=B, R_old=R_old, R_new=R_new, V=V, K_max=int(K_max), reserved=0)
    ws_bytes = gr_beam_select_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = gr_beam_select(dims, _ptr(row_offset_old), _ptr(row_offset_new), _ptr(score_old),
                        _ptr(logits), _ptr(score_new), _ptr(parent), _ptr(token), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if st != GR_OK:
        raise GrAttnError(st, "gr_beam_select")
    return score_new, parent, token


def beam_select_trie(row_offset_old, row_offset_new, score_old, logits, node_old, node_ptr,
                     edge_tok, edge_child, K_max: int, max_fanout: int, *, R_new=None,
                     score_new=None, parent=None, token=None, node_new=None, workspace=None,
                     stream=None):
    """Item-constrained beam selection over a CSR semantic-ID trie
    (include/gr_attn.h).  Returns (score_new, parent, token, node_new)."""
    import torch
    for name, t in (("node_old", node_old), ("node_ptr", node_ptr), ("edge_tok", edge_tok),
                    ("edge_child", edge_child)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device int32 tensor")
    R_old, V = logits.shape
    B = row_offset_old.numel() - 1
    if R_new is None:
        if score_new is None:
            raise ValueError("pass R_new or the output tensors")
        R_new = score_new.numel()
    if node_old.numel() != R_old or edge_tok.numel() != edge_child.numel():
        raise ValueError("node_old or edge tables mismatch")
    dev = logits.device
    if score_new is None:
        score_new = torch.empty(R_new, dtype=torch.float32, device=dev)
    if parent is None:
        parent = torch.empty(R_new, dtype=torch.int32, device=dev)
    if token is None:
        token = torch.empty(R_new, dtype=torch.int32, device=dev)
    if node_new is None:
        node_new = torch.empty(R_new, dtype=torch.int32, device=dev)
    for name, t, dt in (("row_offset_old", row_offset_old, torch.int32),
                        ("row_offset_new", row_offset_new, torch.int32),
                        ("score_old", score_old, torch.float32), ("logits", logits, torch.float32),
                        ("score_new", score_new, torch.float32), ("parent", parent, torch.int32),
                        ("token", token, torch.int32), ("node_new", node_new, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device {dt} tensor")
    dims = SelectDims(B=B, R_old=R_old, R_new=R_new, V=V, K_max=int(K_max), reserved=0)
    trie = SidTrie(node_ptr=_ptr(node_ptr), edge_tok=_ptr(edge_tok), edge_child=_ptr(edge_child),
                   n_nodes=node_ptr.numel() - 1, n_edges=edge_tok.numel(),
                   max_fanout=int(max_fanout), reserved=0)
    ws_bytes = gr_beam_select_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = gr_beam_select_trie(dims, trie, _ptr(row_offset_old), _ptr(row_offset_new),
                             _ptr(score_old), _ptr(logits), _ptr(node_old), _ptr(score_new),
                             _ptr(parent), _ptr(token), _ptr(node_new), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if st != GR_OK:
        raise GrAttnError(st, "gr_beam_select_trie")
    return score_new, parent, token, node_new
