"""Python binding of libgsa, the MI355X (gfx950) Gist Sparse Attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgsa.so`` behind the C ABI declared in ``include/gsa.h``.
PyTorch supplies device memory and the stream. If the library has not been
built, every call raises (there is no fallback path).

Entry points (same names as the C ABI):
  gsa_decode(q, k_cache, v_cache, chunk=, topk=, tail=, ...)
  gsa_decode_varlen(q, k_cache, v_cache, seq_n_raw=, seq_n_gist=, chunk=, topk=, tail=, ...)
  gsa_decode_paged(q, k_pool, v_pool, block_table=, seq_n_raw=, seq_n_gist=, page_chunks=, ...)
  gsa_decode_hier(q, k_cache, v_cache, k_l2, v_l2, chunk=, fanout=, topk1=, topk2=, tail=, ...)
  gsa_decode_levels(q, k_cache, v_cache, k_up, v_up, chunk=, fanout=, topks=, tail=, ...)
  gsa_prefill_blocksparse(q, k_cache, v_cache, chunk=, topk=, window=, q_start=, ...)
  gsa_gist_prefill(q, k_cache, v_cache, chunk=, m_start=, ...)
  gsa_cache_append(k_cache, v_cache, chunk=, n_raw=, n_gist=, k_raw=, v_raw=, k_gist=, v_gist=)

Caches sized for more rows than they hold (to grow in place with
gsa_cache_append) take n_raw= and n_gist= explicitly; their row count is then
the capacity (row_capacity in the C structs).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "GsaError", "lib", "LIB_PATH", "DecodeParams", "HierParams", "PrefillParams", "GistParams",
    "AppendParams", "LevelsParams", "MAX_LEVELS", "GSA_F32", "GSA_BF16", "EXPORTED_SYMBOLS",
    "decode_params", "hier_params", "prefill_params", "gist_params", "append_params", "levels_params",
    "decode_workspace_size", "hier_workspace_size", "prefill_workspace_size", "new_workspace",
    "gsa_decode", "gsa_decode_hier", "gsa_prefill_blocksparse", "gsa_profile_events",
    "gsa_profile_marks", "topk_for_budget", "GIST_SETS", "gsa_gist_prefill", "gsa_cache_append",
    "gsa_decode_levels", "levels_workspace_size", "gsa_decode_varlen", "check_seq_lens",
    "launches", "gsa_decode_noalloc", "PagedParams", "paged_params", "paged_workspace_size",
    "check_pages", "gsa_decode_paged", "gsa_decode_hier_varlen", "check_hier_seq_lens",
    "PrefillVarlenParams", "gsa_prefill_varlen", "check_prefill_seqs", "gsa_decode_levels_varlen",
    "check_levels_seq_lens",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsa.so")
GSA_F32, GSA_BF16 = 0, 1
# gsa_status_t
GSA_OK, GSA_ERR_INVALID_ARG, GSA_ERR_UNSUPPORTED, GSA_ERR_WORKSPACE, GSA_ERR_HIP = 0, 1, 2, 3, 4
EXPORTED_SYMBOLS = (
    "gsa_decode_workspace_size", "gsa_decode",
    "gsa_decode_hier_workspace_size", "gsa_decode_hier",
    "gsa_prefill_workspace_size", "gsa_prefill_blocksparse",
    "gsa_profile_events", "gsa_profile_marks", "gsa_status_string", "gsa_last_error",
    "gsa_topk_for_budget", "gsa_gist_prefill", "gsa_cache_append",
    "gsa_decode_levels_workspace_size", "gsa_decode_levels", "gsa_decode_varlen", "gsa_check_seq_lens",
    "gsa_decode_launches", "gsa_decode_hier_launches", "gsa_decode_levels_launches",
    "gsa_prefill_launches", "gsa_decode_noalloc", "gsa_decode_paged_workspace_size",
    "gsa_decode_paged", "gsa_check_pages", "gsa_decode_hier_varlen", "gsa_check_hier_seq_lens",
    "gsa_prefill_varlen_workspace_size", "gsa_prefill_varlen", "gsa_check_prefill_seqs",
    "gsa_decode_levels_varlen", "gsa_check_levels_seq_lens",
)
MAX_LEVELS = 6

_c_i32, _c_i64, _c_f32, _vp, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_void_p, ctypes.c_size_t)


class DecodeParams(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("n_q_heads", _c_i32), ("n_kv_heads", _c_i32),
                ("head_dim", _c_i32), ("n_raw", _c_i64), ("n_gist", _c_i64),
                ("chunk", _c_i32), ("topk", _c_i32), ("tail", _c_i32), ("scale", _c_f32),
                ("dtype", _c_i32), ("gist_set", _c_i32), ("row_capacity", _c_i64)]


class PagedParams(ctypes.Structure):
    _fields_ = [("base", DecodeParams), ("page_chunks", _c_i32), ("max_pages", _c_i32),
                ("n_pages", _c_i64), ("max_extra", _c_i32)]


class HierParams(ctypes.Structure):
    _fields_ = [("base", DecodeParams), ("fanout", _c_i32), ("topk2", _c_i32)]


class LevelsParams(ctypes.Structure):
    _fields_ = [("base", DecodeParams), ("n_levels", _c_i32), ("fanout", _c_i32),
                ("topk_up", _c_i32 * (MAX_LEVELS - 1))]


class PrefillParams(ctypes.Structure):
    _fields_ = [("n_q_heads", _c_i32), ("n_kv_heads", _c_i32), ("head_dim", _c_i32),
                ("chunk", _c_i32), ("topk", _c_i32), ("window", _c_i32), ("n_raw", _c_i64),
                ("n_gist", _c_i64), ("q_start", _c_i64), ("n_q", _c_i64), ("scale", _c_f32),
                ("dtype", _c_i32), ("row_capacity", _c_i64)]


class PrefillVarlenParams(ctypes.Structure):
    _fields_ = [("base", PrefillParams), ("batch", _c_i32)]


class GistParams(ctypes.Structure):
    _fields_ = [("n_q_heads", _c_i32), ("n_kv_heads", _c_i32), ("head_dim", _c_i32),
                ("chunk", _c_i32), ("n_raw", _c_i64), ("n_gist", _c_i64), ("m_start", _c_i64),
                ("n_q", _c_i64), ("scale", _c_f32), ("dtype", _c_i32), ("row_capacity", _c_i64)]


class AppendParams(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("n_kv_heads", _c_i32), ("head_dim", _c_i32),
                ("chunk", _c_i32), ("n_raw", _c_i64), ("n_gist", _c_i64), ("raw_new", _c_i64),
                ("gist_new", _c_i64), ("row_capacity", _c_i64), ("dtype", _c_i32)]


class GsaError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {message}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise GsaError(-1, "libgsa", f"{LIB_PATH} is missing; build it with "
                           "`python -m decode_gsa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.gsa_decode_workspace_size.argtypes = [P(DecodeParams), P(_sz)]
        L.gsa_decode.argtypes = [P(DecodeParams), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.gsa_decode_hier_workspace_size.argtypes = [P(HierParams), P(_sz)]
        L.gsa_decode_hier.argtypes = [P(HierParams), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _sz, _vp]
        L.gsa_prefill_workspace_size.argtypes = [P(PrefillParams), P(_sz)]
        L.gsa_prefill_blocksparse.argtypes = [P(PrefillParams), _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                              _vp]
        L.gsa_decode_levels_workspace_size.argtypes = [P(LevelsParams), P(_sz)]
        L.gsa_decode_levels.argtypes = [P(LevelsParams), _vp, _vp, _vp, P(_vp), P(_vp), _vp, _vp,
                                         P(_vp), _vp, _vp, _sz, _vp]
        L.gsa_decode_varlen.argtypes = [P(DecodeParams), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _sz, _vp]
        L.gsa_check_seq_lens.argtypes = [P(DecodeParams), P(_c_i32), P(_c_i32)]
        L.gsa_decode_hier_varlen.argtypes = [P(HierParams)] + [_vp] * 11 + [_sz, _vp]
        L.gsa_decode_hier_varlen.restype = _c_i32
        L.gsa_check_hier_seq_lens.argtypes = [P(HierParams), P(_c_i32), P(_c_i32)]
        L.gsa_check_hier_seq_lens.restype = _c_i32
        L.gsa_prefill_varlen_workspace_size.argtypes = [P(PrefillVarlenParams), P(_sz)]
        L.gsa_prefill_varlen_workspace_size.restype = _c_i32
        L.gsa_prefill_varlen.argtypes = [P(PrefillVarlenParams)] + [_vp] * 7 + [_sz, _vp]
        L.gsa_prefill_varlen.restype = _c_i32
        L.gsa_check_prefill_seqs.argtypes = [P(PrefillVarlenParams), P(_c_i32)]
        L.gsa_check_prefill_seqs.restype = _c_i32
        L.gsa_decode_levels_varlen.argtypes = [P(LevelsParams), _vp, _vp, _vp, _vp, _vp, P(_vp), P(_vp), _vp,
                                               _vp, P(_vp), _vp, _vp, _sz, _vp]
        L.gsa_decode_levels_varlen.restype = _c_i32
        L.gsa_check_levels_seq_lens.argtypes = [P(LevelsParams), P(_c_i32), P(_c_i32)]
        L.gsa_check_levels_seq_lens.restype = _c_i32
        L.gsa_gist_prefill.argtypes = [P(GistParams), _vp, _vp, _vp, _vp, _vp]
        L.gsa_cache_append.argtypes = [P(AppendParams), _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.gsa_profile_events.argtypes = [P(_vp), _c_i32]
        L.gsa_profile_marks.argtypes = [P(_c_i32)]
        L.gsa_decode_paged_workspace_size.argtypes = [P(PagedParams), P(_sz)]
        L.gsa_decode_paged_workspace_size.restype = _c_i32
        L.gsa_decode_paged.argtypes = [P(PagedParams)] + [_vp] * 11 + [_sz, _vp]
        L.gsa_decode_paged.restype = _c_i32
        L.gsa_check_pages.argtypes = [P(PagedParams), _vp, _vp, _vp, _vp]
        L.gsa_check_pages.restype = _c_i32
        L.gsa_decode_noalloc.argtypes = [P(DecodeParams), _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.gsa_decode_noalloc.restype = _c_i32
        L.gsa_decode_launches.argtypes = [P(DecodeParams), P(_c_i32)]
        L.gsa_decode_hier_launches.argtypes = [P(HierParams), P(_c_i32)]
        L.gsa_decode_levels_launches.argtypes = [P(LevelsParams), P(_c_i32)]
        L.gsa_prefill_launches.argtypes = [P(PrefillParams), P(_c_i32)]
        for f in ("gsa_decode_workspace_size", "gsa_decode", "gsa_decode_hier_workspace_size",
                  "gsa_decode_hier", "gsa_prefill_workspace_size", "gsa_prefill_blocksparse",
                  "gsa_profile_events", "gsa_profile_marks", "gsa_decode_launches",
                  "gsa_decode_hier_launches", "gsa_decode_levels_launches",
                  "gsa_prefill_launches"):
            getattr(L, f).restype = _c_i32
        L.gsa_topk_for_budget.argtypes = [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32, P(_c_i32)]
        L.gsa_topk_for_budget.restype = _c_i32
        L.gsa_status_string.argtypes = [_c_i32]
        L.gsa_status_string.restype = ctypes.c_char_p
        L.gsa_last_error.argtypes = []
        L.gsa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def gsa_profile_events(handles) -> None:
    """Arm this thread's timing hook with raw hipEvent_t handles (ints); an
    empty sequence disarms it. See gsa_profile_events in include/gsa.h."""
    arr = (_vp * max(1, len(handles)))(*[_vp(h) for h in handles])
    _check(lib().gsa_profile_events(arr, len(handles)), "gsa_profile_events")


def gsa_profile_marks() -> int:
    """Kernel launches + 1 of the last library call on this thread."""
    n = _c_i32(0)
    _check(lib().gsa_profile_marks(ctypes.byref(n)), "gsa_profile_marks")
    return n.value


def launches(p) -> int:
    """Kernel launches a call with these parameters makes (host only): p is a
    DecodeParams, HierParams, LevelsParams or PrefillParams."""
    f = {DecodeParams: "gsa_decode_launches", HierParams: "gsa_decode_hier_launches",
         LevelsParams: "gsa_decode_levels_launches", PrefillParams: "gsa_prefill_launches"}[type(p)]
    n = _c_i32(0)
    _check(getattr(lib(), f)(ctypes.byref(p), ctypes.byref(n)), f)
    return n.value


def _check(status: int, where: str) -> None:
    if status != 0:
        msg = lib().gsa_last_error().decode(errors="replace")
        raise GsaError(status, where, msg or lib().gsa_status_string(status).decode())


# ------------------------------------------------------------ parameters ---

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GSA_BF16
    if t.dtype == torch.float32:
        return GSA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def decode_params(batch, n_q_heads, n_kv_heads, head_dim, n_raw, n_gist, chunk, topk, tail,
                  scale=0.0, dtype=GSA_BF16, gist_set=0, row_capacity=0) -> DecodeParams:
    return DecodeParams(batch, n_q_heads, n_kv_heads, head_dim, n_raw, n_gist, chunk, topk,
                        tail, scale, dtype, gist_set, row_capacity)


def hier_params(base: DecodeParams, fanout: int, topk2: int) -> HierParams:
    return HierParams(base, fanout, topk2)


def levels_params(base: DecodeParams, fanout: int, topk_up) -> LevelsParams:
    """topk_up = [k_2, ..., k_L] (base.topk is k_1)."""
    if not 1 <= len(topk_up) <= MAX_LEVELS - 1:
        raise ValueError(f"2 to {MAX_LEVELS} levels")
    arr = (_c_i32 * (MAX_LEVELS - 1))(*([int(k) for k in topk_up] + [0] * (MAX_LEVELS - 1 - len(topk_up))))
    return LevelsParams(base, len(topk_up) + 1, fanout, arr)


def prefill_params(n_q_heads, n_kv_heads, head_dim, chunk, topk, window, n_raw, n_gist, q_start,
                   n_q, scale=0.0, dtype=GSA_BF16, row_capacity=0) -> PrefillParams:
    return PrefillParams(n_q_heads, n_kv_heads, head_dim, chunk, topk, window, n_raw, n_gist,
                         q_start, n_q, scale, dtype, row_capacity)


def gist_params(n_q_heads, n_kv_heads, head_dim, chunk, n_raw, n_gist, m_start, n_q, scale=0.0,
                dtype=GSA_BF16, row_capacity=0) -> GistParams:
    return GistParams(n_q_heads, n_kv_heads, head_dim, chunk, n_raw, n_gist, m_start, n_q, scale,
                      dtype, row_capacity)


def append_params(batch, n_kv_heads, head_dim, chunk, n_raw, n_gist, raw_new, gist_new,
                  row_capacity, dtype=GSA_BF16) -> AppendParams:
    return AppendParams(batch, n_kv_heads, head_dim, chunk, n_raw, n_gist, raw_new, gist_new,
                        row_capacity, dtype)


def decode_workspace_size(p: DecodeParams) -> int:
    n = _sz(0)
    _check(lib().gsa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "gsa_decode_workspace_size")
    return n.value


def hier_workspace_size(p: HierParams) -> int:
    n = _sz(0)
    _check(lib().gsa_decode_hier_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "gsa_decode_hier_workspace_size")
    return n.value


def levels_workspace_size(p: LevelsParams) -> int:
    n = _sz(0)
    _check(lib().gsa_decode_levels_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "gsa_decode_levels_workspace_size")
    return n.value


def prefill_workspace_size(p: PrefillParams) -> int:
    n = _sz(0)
    _check(lib().gsa_prefill_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "gsa_prefill_workspace_size")
    return n.value


# ------------------------------------------------------------- tensors -----

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _on_stream(stream, device):
    """The call's stream (the current one when None) and a context that makes it
    current: outputs and temporary workspaces are allocated (and zero-filled)
    under it, so they are ordered before the launch and the caching allocator
    reuses them only after the work queued on that stream."""
    import torch
    if torch.device(device).type != "cuda":
        raise ValueError("tensors must live on the GPU")
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s, torch.cuda.stream(s)


def _workspace(ws, nbytes, device):
    """Caller's workspace, or a new zero-filled one (the control words at its
    start must be zero before first use; every call leaves them zero)."""
    import torch
    if ws is not None:
        return ws
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)


def new_workspace(nbytes: int, device="cuda"):
    """A zero-filled device workspace of nbytes, reusable by later calls."""
    import torch
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _geometry(rows: int, chunk: int, n_gist: Optional[int], n_raw: Optional[int]):
    """(N, M, row_capacity) of a cache whose row dimension is `rows`: all rows
    in use unless n_raw is given, in which case `rows` is the capacity."""
    if n_raw is None:
        M = rows // (chunk + 1) if n_gist is None else n_gist
        return rows - M, M, 0
    if n_gist is None:
        raise ValueError("n_raw= needs n_gist= as well")
    return n_raw, n_gist, rows


GIST_SETS = {"all": 0, "selected": 1, "none": 2}


def topk_for_budget(budget: int, n_gist: int, chunk: int, tail: int, gist_set: str = "all") -> int:
    """Fixed-token-budget mode: the largest top-k whose attention set fits
    `budget` tokens (see gsa_topk_for_budget in include/gsa.h)."""
    k = _c_i32(0)
    _check(lib().gsa_topk_for_budget(budget, n_gist, chunk, tail, GIST_SETS[gist_set], ctypes.byref(k)),
           "gsa_topk_for_budget")
    return k.value


def gsa_decode(q, k_cache, v_cache, *, chunk: int, topk: int, tail: int,
               n_gist: Optional[int] = None, scale: float = 0.0, out=None, lse=None,
               sel_idx=None, workspace=None, stream=None, want_lse: bool = True,
               want_sel: bool = True, gist_set: str = "all", n_raw: Optional[int] = None):
    """Single-level GSA decode. q [B,Hq,D]; caches [B,Hkv,R,D] (bf16 or fp32).
    gist_set: "all" (every gist), "selected" (the chosen chunks' gists) or
    "none" -- which gist rows the attention set holds.

    Returns (out [B,Hq,D] fp32, lse [B,Hq] fp32 or None, sel [B,Hkv,k] int32 or None).
    """
    import torch
    B, Hq, D = q.shape
    Hkv, R = k_cache.shape[1], k_cache.shape[2]
    N, M, cap = _geometry(R, chunk, n_gist, n_raw)
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {tuple(GIST_SETS)}")
    p = decode_params(B, Hq, Hkv, D, N, M, chunk, topk, tail, scale, _dtype_code(q),
                      GIST_SETS[gist_set], cap)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache, v_cache must share one dtype")
    if tuple(k_cache.shape) != (B, Hkv, R, D) or tuple(v_cache.shape) != (B, Hkv, R, D):
        raise ValueError("cache shape mismatch")
    dev = q.device
    s, on_s = _on_stream(stream, dev)
    with on_s:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev) if out is None else out
        if lse is None and want_lse:
            lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        if sel_idx is None and want_sel:
            sel_idx = torch.empty(B, Hkv, max(topk, 0), dtype=torch.int32, device=dev)
        ws = _workspace(workspace, decode_workspace_size(p), dev)
        _check(lib().gsa_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                _ptr(lse), _ptr(sel_idx) if topk > 0 else None, _ptr(ws),
                                _nbytes(ws), s.cuda_stream), "gsa_decode")
    return out, lse, sel_idx


def gsa_decode_noalloc(q, k_cache, v_cache, *, chunk: int, topk: int, tail: int, out, lse=None,
                       sel_idx=None, n_gist: Optional[int] = None, n_raw: Optional[int] = None,
                       scale: float = 0.0, stream=None, gist_set: str = "all"):
    """gsa_decode with the library's own scratch as its workspace: nothing is
    allocated, so the outputs are the caller's (out [B,Hq,D] fp32, lse
    [B,Hq] or None, sel_idx [B,Hkv,k] int32 or None)."""
    B, Hq, D = q.shape
    Hkv, R = k_cache.shape[1], k_cache.shape[2]
    N, M, cap = _geometry(R, chunk, n_gist, n_raw)
    p = decode_params(B, Hq, Hkv, D, N, M, chunk, topk, tail, scale, _dtype_code(q),
                      GIST_SETS[gist_set], cap)
    s, _ = _on_stream(stream, q.device)
    _check(lib().gsa_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(out), _ptr(lse), _ptr(sel_idx) if topk > 0 else None,
                                    s.cuda_stream), "gsa_decode_noalloc")
    return out, lse, sel_idx


def paged_params(base: DecodeParams, page_chunks: int, max_pages: int, n_pages: int,
                 max_extra: int = 0) -> PagedParams:
    return PagedParams(base, page_chunks, max_pages, n_pages, max_extra)


def paged_workspace_size(p: PagedParams) -> int:
    n = _sz(0)
    _check(lib().gsa_decode_paged_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "gsa_decode_paged_workspace_size")
    return n.value


def _host_i32(x):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(x.cpu() if hasattr(x, "cpu") else x, dtype=np.int32))
    return a


def check_pages(p: PagedParams, block_table, seq_n_raw, seq_n_gist, extra_rows=None) -> None:
    """Host check of paged inputs (see gsa_check_pages in include/gsa.h)."""
    bt, n, m = _host_i32(block_table), _host_i32(seq_n_raw), _host_i32(seq_n_gist)
    ex = _host_i32(extra_rows) if extra_rows is not None else None
    _check(lib().gsa_check_pages(ctypes.byref(p), bt.ctypes.data, n.ctypes.data, m.ctypes.data,
                                 ex.ctypes.data if ex is not None else None), "gsa_check_pages")


def gsa_decode_paged(q, k_pool, v_pool, *, block_table, seq_n_raw, seq_n_gist, chunk: int, topk: int,
                     tail: int, page_chunks: int, extra_rows=None, n_raw: Optional[int] = None,
                     n_gist: Optional[int] = None, scale: float = 0.0, out=None, lse=None,
                     sel_idx=None, workspace=None, stream=None, want_lse: bool = True,
                     want_sel: bool = True, gist_set: str = "all"):
    """Decode over paged caches (gist_set: as gsa_decode; extra rows are
    attended under every rule). k_pool, v_pool [n_pages, Hkv, P(C+1), D];
    block_table [B, max_pages], seq_n_raw / seq_n_gist [B], extra_rows
    [B, max_extra, 2] (page, row) or None. Host arrays are checked with
    gsa_check_pages and copied to the device; device int32 tensors are used as
    given (then n_raw= and n_gist=, the batch's largest, are required).

    Returns (out [B,Hq,D] fp32, lse [B,Hq] or None, sel [B,Hkv,k] or None).
    """
    import torch
    B, Hq, D = q.shape
    n_pages, Hkv, rpp = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if rpp != page_chunks * (chunk + 1) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("pools must be [n_pages, Hkv, page_chunks * (chunk + 1), D], K and V alike")
    dev = q.device
    on_dev = isinstance(block_table, torch.Tensor) and block_table.is_cuda
    if on_dev:
        if n_raw is None or n_gist is None:
            raise ValueError("device tables need n_raw= and n_gist= (the batch's largest)")
        max_pages = block_table.shape[1]
        max_extra = extra_rows.shape[1] if extra_rows is not None else 0
    else:
        n_h, m_h = _host_i32(seq_n_raw), _host_i32(seq_n_gist)
        bt_h = _host_i32(block_table)
        ex_h = _host_i32(extra_rows) if extra_rows is not None else None
        n_raw = int(n_h.max()) if n_raw is None else n_raw
        n_gist = int(m_h.max()) if n_gist is None else n_gist
        max_pages = bt_h.shape[1]
        max_extra = ex_h.shape[1] if ex_h is not None else 0
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {tuple(GIST_SETS)}")
    base = decode_params(B, Hq, Hkv, D, n_raw, n_gist, chunk, topk, tail, scale, _dtype_code(q),
                         GIST_SETS[gist_set])
    p = paged_params(base, page_chunks, max_pages, n_pages, max_extra)
    if not on_dev:
        check_pages(p, bt_h, n_h, m_h, ex_h)
    s, on_s = _on_stream(stream, dev)
    with on_s:
        if on_dev:
            bt, sn, sm, ex = block_table, seq_n_raw, seq_n_gist, extra_rows
        else:
            bt = torch.from_numpy(bt_h).to(dev)
            sn, sm = torch.from_numpy(n_h).to(dev), torch.from_numpy(m_h).to(dev)
            ex = torch.from_numpy(ex_h).to(dev) if ex_h is not None else None
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev) if out is None else out
        if lse is None and want_lse:
            lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        if sel_idx is None and want_sel:
            sel_idx = torch.empty(B, Hkv, max(topk, 0), dtype=torch.int32, device=dev)
        ws = _workspace(workspace, paged_workspace_size(p), dev)
        _check(lib().gsa_decode_paged(ctypes.byref(p), _ptr(bt), _ptr(sn), _ptr(sm),
                                      _ptr(ex) if max_extra > 0 else None, _ptr(q), _ptr(k_pool),
                                      _ptr(v_pool), _ptr(out), _ptr(lse),
                                      _ptr(sel_idx) if topk > 0 else None, _ptr(ws), _nbytes(ws),
                                      s.cuda_stream), "gsa_decode_paged")
    return out, lse, sel_idx


def check_seq_lens(p: DecodeParams, seq_n_raw, seq_n_gist) -> None:
    """Host check of per-sequence lengths against a call's parameters."""
    n = (_c_i32 * p.batch)(*[int(x) for x in seq_n_raw])
    m = (_c_i32 * p.batch)(*[int(x) for x in seq_n_gist])
    _check(lib().gsa_check_seq_lens(ctypes.byref(p), n, m), "gsa_check_seq_lens")


def gsa_decode_varlen(q, k_cache, v_cache, *, seq_n_raw, seq_n_gist, chunk: int, topk: int,
                      tail: int, n_raw: Optional[int] = None, n_gist: Optional[int] = None,
                      scale: float = 0.0, out=None, lse=None, sel_idx=None, workspace=None,
                      stream=None, want_lse: bool = True, want_sel: bool = True,
                      gist_set: str = "all"):
    """Single-level decode of sequences of different lengths (gist_set: as
    gsa_decode). Caches
    [B,Hkv,cap,D]: sequence b uses its first seq_n_raw[b] + seq_n_gist[b] rows.

    seq_n_raw / seq_n_gist: host sequences (checked with gsa_check_seq_lens,
    then copied to the device) or device int32 tensors [B], used as given
    (then n_raw= and n_gist=, the batch's largest values, are required).
    Returns (out, lse, sel) as gsa_decode.
    """
    import torch
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    on_dev = isinstance(seq_n_raw, torch.Tensor) and seq_n_raw.is_cuda
    if on_dev:
        if n_raw is None or n_gist is None:
            raise ValueError("device length arrays need n_raw= and n_gist= (the batch's largest)")
        sn, sm = seq_n_raw, seq_n_gist
    else:
        hn = [int(x) for x in (seq_n_raw.tolist() if hasattr(seq_n_raw, "tolist") else seq_n_raw)]
        hm = [int(x) for x in (seq_n_gist.tolist() if hasattr(seq_n_gist, "tolist") else seq_n_gist)]
        if len(hn) != B or len(hm) != B:
            raise ValueError("one length per sequence")
        n_raw = max(hn) if n_raw is None else n_raw
        n_gist = max(hm) if n_gist is None else n_gist
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {tuple(GIST_SETS)}")
    p = decode_params(B, Hq, Hkv, D, n_raw, n_gist, chunk, topk, tail, scale, _dtype_code(q),
                      GIST_SETS[gist_set], cap)
    if not on_dev:
        check_seq_lens(p, hn, hm)
    s, on_s = _on_stream(stream, dev)
    with on_s:
        if not on_dev:
            sn = torch.tensor(hn, dtype=torch.int32, device=dev)
            sm = torch.tensor(hm, dtype=torch.int32, device=dev)
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev) if out is None else out
        if lse is None and want_lse:
            lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        if sel_idx is None and want_sel:
            sel_idx = torch.empty(B, Hkv, max(topk, 0), dtype=torch.int32, device=dev)
        ws = _workspace(workspace, decode_workspace_size(p), dev)
        _check(lib().gsa_decode_varlen(ctypes.byref(p), _ptr(sn), _ptr(sm), _ptr(q), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(out), _ptr(lse),
                                       _ptr(sel_idx) if topk > 0 else None, _ptr(ws), _nbytes(ws),
                                       s.cuda_stream), "gsa_decode_varlen")
    return out, lse, sel_idx


def gsa_decode_hier(q, k_cache, v_cache, k_l2, v_l2, *, chunk: int, fanout: int, topk1: int,
                    topk2: int, tail: int, n_gist: Optional[int] = None, scale: float = 0.0,
                    out=None, lse=None, sel2=None, sel1=None, workspace=None, stream=None,
                    want_lse: bool = True, want_sel: bool = True, n_raw: Optional[int] = None,
                    gist_set: str = "all"):
    """Two-level (gist-of-gist) decode. k_l2, v_l2 [B,Hkv,M2,D]. gist_set:
    which gists are attended ("all"; "selected": the chosen chunks'; "none").

    Returns (out, lse, sel2 [B,Hkv,k2], sel1 [B,Hkv,k1]).
    """
    import torch
    B, Hq, D = q.shape
    Hkv, R = k_cache.shape[1], k_cache.shape[2]
    N, M, cap = _geometry(R, chunk, n_gist, n_raw)
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {tuple(GIST_SETS)}")
    base = decode_params(B, Hq, Hkv, D, N, M, chunk, topk1, tail, scale, _dtype_code(q),
                         gist_set=GIST_SETS[gist_set], row_capacity=cap)
    p = hier_params(base, fanout, topk2)
    dev = q.device
    s, on_s = _on_stream(stream, dev)
    with on_s:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev) if out is None else out
        if lse is None and want_lse:
            lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        if want_sel:
            if sel2 is None:
                sel2 = torch.empty(B, Hkv, max(topk2, 0), dtype=torch.int32, device=dev)
            if sel1 is None:
                sel1 = torch.empty(B, Hkv, max(topk1, 0), dtype=torch.int32, device=dev)
        ws = _workspace(workspace, hier_workspace_size(p), dev)
        _check(lib().gsa_decode_hier(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(k_l2), _ptr(v_l2), _ptr(out), _ptr(lse),
                                     _ptr(sel2) if topk2 > 0 else None,
                                     _ptr(sel1) if topk1 > 0 else None, _ptr(ws), _nbytes(ws),
                                     s.cuda_stream), "gsa_decode_hier")
    return out, lse, sel2, sel1


def check_hier_seq_lens(p: HierParams, seq_n_raw, seq_n_gist) -> None:
    """Host check of per-sequence lengths against a two-level call's parameters."""
    n = (_c_i32 * p.base.batch)(*[int(x) for x in seq_n_raw])
    m = (_c_i32 * p.base.batch)(*[int(x) for x in seq_n_gist])
    _check(lib().gsa_check_hier_seq_lens(ctypes.byref(p), n, m), "gsa_check_hier_seq_lens")


def gsa_decode_hier_varlen(q, k_cache, v_cache, k_l2, v_l2, *, seq_n_raw, seq_n_gist, chunk: int,
                           fanout: int, topk1: int, topk2: int, tail: int, n_raw: Optional[int] = None,
                           n_gist: Optional[int] = None, scale: float = 0.0, out=None, lse=None,
                           sel2=None, sel1=None, workspace=None, stream=None, want_lse: bool = True,
                           want_sel: bool = True, gist_set: str = "all"):
    """Two-level decode of sequences of different lengths. Caches
    [B,Hkv,cap,D] (sequence b: its first seq_n_raw[b] + seq_n_gist[b] rows);
    k_l2, v_l2 [B,Hkv,M2,D] with M2 = n_gist // fanout (sequence b: its first
    seq_n_gist[b] // fanout rows).

    seq_n_raw / seq_n_gist: host sequences (checked with
    gsa_check_hier_seq_lens, then copied to the device) or device int32
    tensors [B], used as given (then n_raw= and n_gist=, the batch's largest
    values, are required). Returns (out, lse, sel2, sel1) as gsa_decode_hier.
    """
    import torch
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    on_dev = isinstance(seq_n_raw, torch.Tensor) and seq_n_raw.is_cuda
    if on_dev:
        if n_raw is None or n_gist is None:
            raise ValueError("device length arrays need n_raw= and n_gist= (the batch's largest)")
        sn, sm = seq_n_raw, seq_n_gist
    else:
        hn = [int(x) for x in (seq_n_raw.tolist() if hasattr(seq_n_raw, "tolist") else seq_n_raw)]
        hm = [int(x) for x in (seq_n_gist.tolist() if hasattr(seq_n_gist, "tolist") else seq_n_gist)]
        if len(hn) != B or len(hm) != B:
            raise ValueError("one length per sequence")
        n_raw = max(hn) if n_raw is None else n_raw
        n_gist = max(hm) if n_gist is None else n_gist
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {tuple(GIST_SETS)}")
    base = decode_params(B, Hq, Hkv, D, n_raw, n_gist, chunk, topk1, tail, scale, _dtype_code(q),
                         gist_set=GIST_SETS[gist_set], row_capacity=cap)
    p = hier_params(base, fanout, topk2)
    if k_l2.shape[2] != n_gist // fanout:
        raise ValueError(f"level-2 arrays hold {k_l2.shape[2]} rows per slab, expected {n_gist // fanout}")
    if not on_dev:
        check_hier_seq_lens(p, hn, hm)
    s, on_s = _on_stream(stream, dev)
    with on_s:
        if not on_dev:
            sn = torch.tensor(hn, dtype=torch.int32, device=dev)
            sm = torch.tensor(hm, dtype=torch.int32, device=dev)
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev) if out is None else out
        if lse is None and want_lse:
            lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        if want_sel:
            if sel2 is None:
                sel2 = torch.empty(B, Hkv, max(topk2, 0), dtype=torch.int32, device=dev)
            if sel1 is None:
                sel1 = torch.empty(B, Hkv, max(topk1, 0), dtype=torch.int32, device=dev)
        ws = _workspace(workspace, hier_workspace_size(p), dev)
        _check(lib().gsa_decode_hier_varlen(ctypes.byref(p), _ptr(sn), _ptr(sm), _ptr(q), _ptr(k_cache),
                                            _ptr(v_cache), _ptr(k_l2), _ptr(v_l2), _ptr(out), _ptr(lse),
                                            _ptr(sel2) if topk2 > 0 and want_sel else None,
                                            _ptr(sel1) if topk1 > 0 and want_sel else None, _ptr(ws),
                                            _nbytes(ws), s.cuda_stream), "gsa_decode_hier_varlen")
    return out, lse, sel2, sel1


def gsa_decode_levels(q, k_cache, v_cache, k_up, v_up, *, chunk: int, fanout: int, topks,
                      tail: int, n_gist: Optional[int] = None, n_raw: Optional[int] = None,
                      scale: float = 0.0, out=None, lse=None, workspace=None, stream=None,
                      want_lse: bool = True, want_sel: bool = True, gist_set: str = "all"):
    """L-level decode. k_up, v_up: [level 2, ..., level L] arrays [B,Hkv,M_l,D];
    topks = [k_1, ..., k_L].

    Returns (out [B,Hq,D] fp32, lse [B,Hq] or None, sels [sel_1 [B,Hkv,k_1], ...,
    sel_L] or None).
    """
    import torch
    B, Hq, D = q.shape
    Hkv, R = k_cache.shape[1], k_cache.shape[2]
    N, M, cap = _geometry(R, chunk, n_gist, n_raw)
    topks = [int(k) for k in topks]
    if len(k_up) != len(topks) - 1 or len(v_up) != len(topks) - 1:
        raise ValueError("one k per level and one array pair per level above the first")
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {tuple(GIST_SETS)}")
    base = decode_params(B, Hq, Hkv, D, N, M, chunk, topks[0], tail, scale, _dtype_code(q),
                         gist_set=GIST_SETS[gist_set], row_capacity=cap)
    p = levels_params(base, fanout, topks[1:])
    dev = q.device
    s, on_s = _on_stream(stream, dev)
    with on_s:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev) if out is None else out
        if lse is None and want_lse:
            lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        sels = ([torch.empty(B, Hkv, max(k, 0), dtype=torch.int32, device=dev) for k in topks]
                if want_sel else None)
        n_up = len(k_up)
        kp = (_vp * n_up)(*[_ptr(t) if t.numel() else None for t in k_up])
        vp = (_vp * n_up)(*[_ptr(t) if t.numel() else None for t in v_up])
        sp = (_vp * n_up)(*[_ptr(t) if t.numel() else None for t in sels[1:]]) if want_sel else None
        ws = _workspace(workspace, levels_workspace_size(p), dev)
        _check(lib().gsa_decode_levels(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), kp,
                                       vp, _ptr(out), _ptr(lse), sp,
                                       _ptr(sels[0]) if want_sel and topks[0] > 0 else None,
                                       _ptr(ws), _nbytes(ws), s.cuda_stream), "gsa_decode_levels")
    return out, lse, sels


def check_levels_seq_lens(p: LevelsParams, seq_n_raw, seq_n_gist) -> None:
    """Host check of per-sequence lengths against an L-level call's parameters."""
    n = (_c_i32 * p.base.batch)(*[int(x) for x in seq_n_raw])
    m = (_c_i32 * p.base.batch)(*[int(x) for x in seq_n_gist])
    _check(lib().gsa_check_levels_seq_lens(ctypes.byref(p), n, m), "gsa_check_levels_seq_lens")


def gsa_decode_levels_varlen(q, k_cache, v_cache, k_up, v_up, *, seq_n_raw, seq_n_gist, chunk: int,
                             fanout: int, topks, tail: int, n_raw: Optional[int] = None,
                             n_gist: Optional[int] = None, scale: float = 0.0, out=None, lse=None,
                             workspace=None, stream=None, want_lse: bool = True, want_sel: bool = True,
                             gist_set: str = "all"):
    """L-level decode of sequences of different lengths. Caches [B,Hkv,cap,D]
    (sequence b: its first seq_n_raw[b] + seq_n_gist[b] rows); k_up, v_up:
    level l's arrays [B,Hkv,M_l,D] with M_l = n_gist // fanout^(l-1) (sequence
    b: its first seq_n_gist[b] // fanout^(l-1) rows). seq_n_raw / seq_n_gist:
    host sequences (checked with gsa_check_levels_seq_lens) or device int32
    tensors [B] (then n_raw= and n_gist=, the batch's largest, are required).
    Returns (out, lse, sels) as gsa_decode_levels.
    """
    import torch
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    on_dev = isinstance(seq_n_raw, torch.Tensor) and seq_n_raw.is_cuda
    if on_dev:
        if n_raw is None or n_gist is None:
            raise ValueError("device length arrays need n_raw= and n_gist= (the batch's largest)")
        sn, sm = seq_n_raw, seq_n_gist
    else:
        hn = [int(x) for x in (seq_n_raw.tolist() if hasattr(seq_n_raw, "tolist") else seq_n_raw)]
        hm = [int(x) for x in (seq_n_gist.tolist() if hasattr(seq_n_gist, "tolist") else seq_n_gist)]
        if len(hn) != B or len(hm) != B:
            raise ValueError("one length per sequence")
        n_raw = max(hn) if n_raw is None else n_raw
        n_gist = max(hm) if n_gist is None else n_gist
    topks = [int(k) for k in topks]
    if len(k_up) != len(topks) - 1 or len(v_up) != len(topks) - 1:
        raise ValueError("one k per level and one array pair per level above the first")
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {tuple(GIST_SETS)}")
    base = decode_params(B, Hq, Hkv, D, n_raw, n_gist, chunk, topks[0], tail, scale, _dtype_code(q),
                         gist_set=GIST_SETS[gist_set], row_capacity=cap)
    p = levels_params(base, fanout, topks[1:])
    if not on_dev:
        check_levels_seq_lens(p, hn, hm)
    s, on_s = _on_stream(stream, dev)
    with on_s:
        if not on_dev:
            sn = torch.tensor(hn, dtype=torch.int32, device=dev)
            sm = torch.tensor(hm, dtype=torch.int32, device=dev)
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev) if out is None else out
        if lse is None and want_lse:
            lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        sels = ([torch.empty(B, Hkv, max(k, 0), dtype=torch.int32, device=dev) for k in topks]
                if want_sel else None)
        n_up = len(k_up)
        kp = (_vp * n_up)(*[_ptr(t) if t.numel() else None for t in k_up])
        vp = (_vp * n_up)(*[_ptr(t) if t.numel() else None for t in v_up])
        sp = (_vp * n_up)(*[_ptr(t) if t.numel() else None for t in sels[1:]]) if want_sel else None
        ws = _workspace(workspace, levels_workspace_size(p), dev)
        _check(lib().gsa_decode_levels_varlen(ctypes.byref(p), _ptr(sn), _ptr(sm), _ptr(q), _ptr(k_cache),
                                              _ptr(v_cache), kp, vp, _ptr(out), _ptr(lse), sp,
                                              _ptr(sels[0]) if want_sel and topks[0] > 0 else None,
                                              _ptr(ws), _nbytes(ws), s.cuda_stream), "gsa_decode_levels_varlen")
    return out, lse, sels


def gsa_prefill_blocksparse(q, k_cache, v_cache, *, chunk: int, topk: int, window: int,
                            q_start: int, n_gist: Optional[int] = None, scale: float = 0.0,
                            out=None, sel=None, workspace=None, stream=None,
                            want_sel: bool = True, n_raw: Optional[int] = None):
    """Causal block-sparse prefill. q [Hq,n_q,D]; caches [Hkv,R,D] (bf16).

    Returns (out [Hq,n_q,D] fp32, sel [Hkv,n_q,k] int32 or None).
    """
    import torch
    Hq, n_q, D = q.shape
    Hkv, R = k_cache.shape[0], k_cache.shape[1]
    N, M, cap = _geometry(R, chunk, n_gist, n_raw)
    p = prefill_params(Hq, Hkv, D, chunk, topk, window, N, M, q_start, n_q, scale,
                       _dtype_code(q), cap)
    dev = q.device
    s, on_s = _on_stream(stream, dev)
    with on_s:
        out = torch.empty(Hq, n_q, D, dtype=torch.float32, device=dev) if out is None else out
        if sel is None and want_sel:
            sel = torch.empty(Hkv, n_q, max(topk, 0), dtype=torch.int32, device=dev)
        ws = _workspace(workspace, prefill_workspace_size(p), dev)
        _check(lib().gsa_prefill_blocksparse(ctypes.byref(p), _ptr(q), _ptr(k_cache),
                                             _ptr(v_cache), _ptr(out),
                                             _ptr(sel) if topk > 0 else None, _ptr(ws),
                                             _nbytes(ws), s.cuda_stream),
               "gsa_prefill_blocksparse")
    return out, sel


def check_prefill_seqs(p: PrefillVarlenParams, seqs) -> None:
    """Host check of a batched prefill's per-sequence (n_raw, n_gist, q_start, n_q)."""
    flat = [int(x) for row in seqs for x in row]
    arr = (_c_i32 * len(flat))(*flat)
    _check(lib().gsa_check_prefill_seqs(ctypes.byref(p), arr), "gsa_check_prefill_seqs")


def gsa_prefill_varlen(q, k_cache, v_cache, *, seqs, chunk: int, topk: int, window: int,
                       n_raw: Optional[int] = None, n_gist: Optional[int] = None, scale: float = 0.0,
                       out=None, sel=None, workspace=None, stream=None, want_sel: bool = True):
    """Causal block-sparse prefill of B sequences of different lengths in one
    call. q [B,Hq,n_q,D] (sequence b's query i at position q_start_b + i in
    row i); caches [B,Hkv,R,D] (bf16).

    seqs: host rows (n_raw, n_gist, q_start, n_q) per sequence (checked with
    gsa_check_prefill_seqs, then copied to the device) or a device int32
    tensor [B, 4] used as given (then n_raw= and n_gist=, the batch's
    largest, are required). Returns (out [B,Hq,n_q,D] fp32, sel [B,Hkv,n_q,k]
    int32 or None); rows past a sequence's n_q are not written.
    """
    import torch
    B, Hq, n_q, D = q.shape
    Hkv, R = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    on_dev = isinstance(seqs, torch.Tensor) and seqs.is_cuda
    if on_dev:
        if n_raw is None or n_gist is None:
            raise ValueError("a device seqs array needs n_raw= and n_gist= (the batch's largest)")
        sd = seqs
    else:
        rows = [[int(x) for x in r] for r in (seqs.tolist() if hasattr(seqs, "tolist") else seqs)]
        if len(rows) != B or any(len(r) != 4 for r in rows):
            raise ValueError("one (n_raw, n_gist, q_start, n_q) row per sequence")
        n_raw = max(r[0] for r in rows) if n_raw is None else n_raw
        n_gist = max(r[1] for r in rows) if n_gist is None else n_gist
    base = prefill_params(Hq, Hkv, D, chunk, topk, window, n_raw, n_gist, 0, n_q, scale,
                          _dtype_code(q), R)
    p = PrefillVarlenParams(base, B)
    if not on_dev:
        check_prefill_seqs(p, rows)
    nbytes = _sz(0)
    _check(lib().gsa_prefill_varlen_workspace_size(ctypes.byref(p), ctypes.byref(nbytes)),
           "gsa_prefill_varlen_workspace_size")
    s, on_s = _on_stream(stream, dev)
    with on_s:
        if not on_dev:
            sd = torch.tensor(rows, dtype=torch.int32, device=dev)
        out = torch.empty(B, Hq, n_q, D, dtype=torch.float32, device=dev) if out is None else out
        if sel is None and want_sel:
            sel = torch.empty(B, Hkv, n_q, max(topk, 0), dtype=torch.int32, device=dev)
        ws = _workspace(workspace, nbytes.value, dev)
        _check(lib().gsa_prefill_varlen(ctypes.byref(p), _ptr(sd), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(out), _ptr(sel) if topk > 0 and want_sel else None, _ptr(ws),
                                        _nbytes(ws), s.cuda_stream), "gsa_prefill_varlen")
    return out, sel


def gsa_gist_prefill(q, k_cache, v_cache, *, chunk: int, m_start: int,
                     n_gist: Optional[int] = None, n_raw: Optional[int] = None, scale: float = 0.0,
                     out=None, stream=None):
    """Gist tokens of chunks [m_start, m_start + n_q) of one sequence under the
    gist causal mask. q [Hq,n_q,D]; caches [Hkv,R,D] (bf16).

    Returns out [Hq,n_q,D] fp32.
    """
    import torch
    Hq, n_q, D = q.shape
    Hkv, R = k_cache.shape[0], k_cache.shape[1]
    N, M, cap = _geometry(R, chunk, n_gist, n_raw)
    p = gist_params(Hq, Hkv, D, chunk, N, M, m_start, n_q, scale, _dtype_code(q), cap)
    dev = q.device
    s, on_s = _on_stream(stream, dev)
    with on_s:
        out = torch.empty(Hq, n_q, D, dtype=torch.float32, device=dev) if out is None else out
        _check(lib().gsa_gist_prefill(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(out), s.cuda_stream), "gsa_gist_prefill")
    return out


def gsa_cache_append(k_cache, v_cache, *, chunk: int, n_raw: int, n_gist: int, k_raw=None,
                     v_raw=None, k_gist=None, v_gist=None, stream=None) -> None:
    """Write new raw rows (positions n_raw, n_raw + 1, ...) and new gist rows
    (chunks n_gist, n_gist + 1, ...) into their interleaved slots.

    Caches [B,Hkv,cap,D] or [Hkv,cap,D] (one sequence); k_raw, v_raw
    [..., n_new, D] and k_gist, v_gist [..., g_new, D] with the caches' leading
    dimensions and dtype (None: nothing of that kind).
    """
    lead = tuple(k_cache.shape[:-2])
    cap, D = k_cache.shape[-2], k_cache.shape[-1]
    if len(lead) not in (1, 2) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [B,Hkv,cap,D] or [Hkv,cap,D], K and V alike")
    B, Hkv = (1, lead[0]) if len(lead) == 1 else lead

    def rows(a, b, what):
        if (a is None) != (b is None):
            raise ValueError(f"give both k_{what} and v_{what} or neither")
        if a is None:
            return 0
        if tuple(a.shape[:-2]) != lead or a.shape[-1] != D or tuple(b.shape) != tuple(a.shape):
            raise ValueError(f"k_{what} / v_{what} shape mismatch with the caches")
        if a.dtype != k_cache.dtype or b.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
            raise TypeError("all rows and caches must share one dtype")
        return a.shape[-2]

    n_new, g_new = rows(k_raw, v_raw, "raw"), rows(k_gist, v_gist, "gist")
    p = append_params(B, Hkv, D, chunk, n_raw, n_gist, n_new, g_new, cap, _dtype_code(k_cache))
    _check(lib().gsa_cache_append(ctypes.byref(p), _ptr(k_raw) if n_new else None,
                                  _ptr(v_raw) if n_new else None, _ptr(k_gist) if g_new else None,
                                  _ptr(v_gist) if g_new else None, _ptr(k_cache), _ptr(v_cache),
                                  _on_stream(stream, k_cache.device)[0].cuda_stream),
           "gsa_cache_append")

