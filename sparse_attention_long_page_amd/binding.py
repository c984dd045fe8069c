"""Thin ctypes binding over libsparse_attn.so (include/sparse_attn.h).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  torch provides device memory (outputs, workspaces) and the
current stream.  The functions keep the C names.  A missing library is built
once with hipcc; if that is impossible the import fails loudly -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int32, c_size_t, c_void_p
from typing import Optional

import torch

from . import build as _build

SA_OK = 0
SA_ERR_INVALID_ARGUMENT = 1
SA_ERR_UNSUPPORTED = 2
SA_ERR_WORKSPACE_TOO_SMALL = 3
SA_ERR_DEVICE = 4
SA_ERR_DATA = 5
SA_DTYPE_BF16 = 0
SA_DTYPE_FP32 = 1
SA_DTYPE_FP8_E4M3 = 2
SA_SEL_PER_KV_HEAD = 0
SA_SEL_PER_Q_HEAD = 1
SA_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = [
    "sa_page_summary", "sa_select_pages_workspace_size", "sa_select_pages",
    "sa_sparse_decode_workspace_size", "sa_sparse_decode", "sa_sparse_decode_noalloc", "sa_select_decode",
    "sa_block_sparse_prefill_workspace_size", "sa_block_sparse_prefill", "sa_prefill_block_mask",
    "sa_page_value_summary", "sa_prefill_mean_correction_workspace_size", "sa_prefill_mean_correction",
    "sa_head_page_mass_workspace_size", "sa_head_page_mass", "sa_autotune_tiers_workspace_size", "sa_autotune_tiers",
    "sa_ambient_head_mask", "sa_set_debug_validate",
    "sa_status_string", "sa_last_error_message", "sa_version",
]


class sa_paged_kv(ctypes.Structure):
    _fields_ = [("k_pool", c_void_p), ("v_pool", c_void_p), ("block_table", c_void_p),
                ("seq_lens", c_void_p), ("n_phys_pages", c_int32), ("n_kv_heads", c_int32),
                ("page_size", c_int32), ("d_qk", c_int32), ("d_v", c_int32), ("max_pages", c_int32),
                ("dtype", c_int), ("k_scale", c_void_p), ("v_scale", c_void_p)]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return _build.LIB


def load_library(build_if_missing: bool = True) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        if not build_if_missing:
            raise ImportError(f"{_build.LIB} is not built")
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    P = c_void_p
    sig = {
        "sa_page_summary": (c_int, [P, c_int32, c_int32, P, P]),
        "sa_select_pages_workspace_size": (c_size_t, [c_int32, c_int32, c_int32]),
        "sa_select_pages": (c_int, [P, c_int32, P, c_int32, c_int32, P, c_int32, P, c_int32, c_int, c_int32, c_int32,
                                    c_int32, c_int32, P, c_int32, P, P, P, P, c_size_t, P]),
        "sa_sparse_decode_workspace_size": (c_size_t, [P, c_int32, c_int32, c_int32, c_int32, c_int, c_int32]),
        "sa_sparse_decode": (c_int, [P, c_int32, P, c_int32, c_int32, P, P, c_int32, c_int, P, P, c_float,
                                     c_int32, P, P, P, c_size_t, P]),
        "sa_sparse_decode_noalloc": (c_int, [P, c_int32, P, c_int32, c_int32, P, P, c_int32, c_int, P, P, c_float,
                                             c_int32, P, P, P]),
        "sa_select_decode": (c_int, [P, c_int32, P, c_int32, c_int32, P, c_int32, c_int32, c_int32, c_int32, P,
                                     c_int32, P, c_float, P, P, P]),
        "sa_block_sparse_prefill_workspace_size": (c_size_t, [P, c_int32, c_int32, c_int32]),
        "sa_block_sparse_prefill": (c_int, [P, c_int32, P, c_int32, c_int32, c_int32, P, c_int32, c_int32, P, P,
                                            c_float, P, P, P, c_size_t, P]),
        "sa_prefill_block_mask": (c_int, [P, c_int32, P, c_int32, c_int32, c_int32, P, c_int32, c_int32, c_float,
                                          c_int32, c_float, P, P]),
        "sa_page_value_summary": (c_int, [P, c_int32, c_int32, P, P]),
        "sa_prefill_mean_correction_workspace_size": (c_size_t, [P, c_int32]),
        "sa_prefill_mean_correction": (c_int, [P, c_int32, P, c_int32, c_int32, c_int32, P, P, c_int32, P, P,
                                               c_float, P, P, P, c_size_t, P]),
        "sa_head_page_mass_workspace_size": (c_size_t, [P, c_int32, c_int32, c_int32]),
        "sa_head_page_mass": (c_int, [P, c_int32, P, c_int32, c_int32, P, c_float, P, P, c_size_t, P]),
        "sa_autotune_tiers_workspace_size": (c_size_t, [P, c_int32, c_int32]),
        "sa_autotune_tiers": (c_int, [P, c_int32, c_int32, c_int32, P, P, c_int32, c_int32, c_int32, c_int32, P,
                                      c_int32, P, c_int32, P, P, P, c_size_t, P]),
        "sa_ambient_head_mask": (c_int, [P, c_int32, c_int32, P, P, c_int32, P, P, c_int32, P, P]),
        "sa_set_debug_validate": (c_int, [c_int]),
        "sa_status_string": (ctypes.c_char_p, [c_int]),
        "sa_last_error_message": (ctypes.c_char_p, []),
        "sa_version": (c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    return load_library().sa_status_string(s).decode()


def _check(status: int):
    if status != SA_OK:
        msg = load_library().sa_last_error_message().decode()
        raise SparseAttnError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SA_DTYPE_BF16
    if t.dtype == torch.float32:
        return SA_DTYPE_FP32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return SA_DTYPE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


class PagedKV:
    """Holds the paged cache tensors and the matching C descriptor.  FP8 pools
    (uint8 or float8_e4m3fn E4M3 bytes) come with k_scale / v_scale
    [n_phys][n_kv_heads] fp32; queries and outputs are then bf16."""

    def __init__(self, k_pool: torch.Tensor, v_pool: Optional[torch.Tensor], block_table: torch.Tensor,
                 seq_lens: torch.Tensor, d_v: Optional[int] = None, k_scale: Optional[torch.Tensor] = None,
                 v_scale: Optional[torch.Tensor] = None):
        for t in (k_pool, v_pool, block_table, seq_lens, k_scale, v_scale):
            if t is not None and not t.is_contiguous():
                raise ValueError("paged cache tensors must be contiguous")
        if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
            raise TypeError("block_table and seq_lens must be int32")
        self.k_pool, self.v_pool, self.block_table, self.seq_lens = k_pool, v_pool, block_table, seq_lens
        n_phys, n_kv, P, d_qk = k_pool.shape
        if v_pool is not None:
            d_v = v_pool.shape[2]
        elif d_v is None:
            d_v = 512
        code = _dtype_code(k_pool)
        if code == SA_DTYPE_FP8_E4M3 and (k_scale is None or v_scale is None):
            raise ValueError("FP8 pools need k_scale and v_scale")
        self.k_scale, self.v_scale = k_scale, v_scale
        self.c = sa_paged_kv(k_pool.data_ptr(), None if v_pool is None else v_pool.data_ptr(),
                             block_table.data_ptr(), seq_lens.data_ptr(), n_phys, n_kv, P, d_qk, d_v,
                             block_table.shape[1], code,
                             None if k_scale is None else k_scale.data_ptr(),
                             None if v_scale is None else v_scale.data_ptr())
        self.batch = block_table.shape[0]
        self.n_kv_heads, self.page_size, self.d_qk, self.d_v = n_kv, P, d_qk, d_v
        self.max_pages = block_table.shape[1]
        self.device = k_pool.device
        self.dtype = torch.bfloat16 if code == SA_DTYPE_FP8_E4M3 else k_pool.dtype   # of queries and outputs

    @property
    def ref(self):
        return ctypes.byref(self.c)


def sa_page_summary(kv: PagedKV, last_pages: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.full((kv.c.n_phys_pages, kv.n_kv_heads, kv.d_qk), float("nan"), dtype=torch.float32,
                         device=kv.device)
    _check(load_library().sa_page_summary(kv.ref, kv.batch, last_pages, _ptr(out), _stream(kv.device)))
    return out


def sa_select_pages_workspace_size(batch: int, n_sel: int, max_pages: int) -> int:
    return load_library().sa_select_pages_workspace_size(batch, n_sel, max_pages)


def sa_select_pages(kv: PagedKV, *, n_q_heads: int, mode: int, sink_pages: int, window_pages: int, top_k: int,
                    q: Optional[torch.Tensor] = None, page_summary: Optional[torch.Tensor] = None,
                    scores: Optional[torch.Tensor] = None, critical_k: Optional[int] = None,
                    list_stride: Optional[int] = None, scores_out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, out=None, refresh_newest_page: bool = False):
    """Returns (page_lists [B][n_sel][list_stride] int32, page_counts, critical_counts or None).
    refresh_newest_page: first rewrite page_summary for each sequence's newest page
    (as sa_page_summary(kv, last_pages=1) would), then score with it."""
    B = kv.batch
    n_sel = kv.n_kv_heads if mode == SA_SEL_PER_KV_HEAD else n_q_heads
    if list_stride is None:
        list_stride = min(kv.max_pages, sink_pages + window_pages + top_k)
        list_stride = max(list_stride, 1)
    if out is None:
        lists = torch.full((B, n_sel, list_stride), -1, dtype=torch.int32, device=kv.device)
        counts = torch.zeros((B, n_sel), dtype=torch.int32, device=kv.device)
        ccounts = torch.zeros((B, n_sel), dtype=torch.int32, device=kv.device) if critical_k is not None else None
    else:
        lists, counts, ccounts = out
    q_tokens = q.shape[1] if q is not None else 1
    scores_stride = scores.shape[-1] if scores is not None else 0
    if workspace is None and scores is None:
        nbytes = sa_select_pages_workspace_size(B, n_sel, kv.max_pages)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=kv.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(load_library().sa_select_pages(
        kv.ref, B, _ptr(q), q_tokens, n_q_heads, _ptr(page_summary), 1 if refresh_newest_page else 0, _ptr(scores),
        scores_stride, mode,
        sink_pages, window_pages, top_k, critical_k if critical_k is not None else 0, _ptr(lists),
        list_stride, _ptr(counts), _ptr(ccounts), _ptr(scores_out), _ptr(workspace), ws_bytes,
        _stream(kv.device)))
    return lists, counts, ccounts


def sa_sparse_decode_workspace_size(kv: PagedKV, q_tokens: int, n_q_heads: int, list_stride: int, mode: int,
                                    num_splits: int = 0) -> int:
    return load_library().sa_sparse_decode_workspace_size(kv.ref, kv.batch, q_tokens, n_q_heads, list_stride,
                                                          mode, num_splits)


def sa_sparse_decode(kv: PagedKV, q: torch.Tensor, page_lists: torch.Tensor, page_counts: torch.Tensor, *,
                     mode: int, sm_scale: float, critical_counts: Optional[torch.Tensor] = None,
                     ambient_head_mask: Optional[torch.Tensor] = None, num_splits: int = 0,
                     out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, want_lse: bool = True):
    """Returns (out [B][T][Hq][d_v], lse [B][T][Hq] fp32 or None)."""
    B, T, Hq, _ = q.shape
    list_stride = page_lists.shape[-1]
    if out is None:
        out = torch.empty((B, T, Hq, kv.d_v), dtype=kv.dtype, device=kv.device)
    if out_lse is None and want_lse:
        out_lse = torch.empty((B, T, Hq), dtype=torch.float32, device=kv.device)
    if workspace is None:
        nbytes = sa_sparse_decode_workspace_size(kv, T, Hq, list_stride, mode, num_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=kv.device)
    _check(load_library().sa_sparse_decode(
        kv.ref, B, _ptr(q), T, Hq, _ptr(page_lists), _ptr(page_counts), list_stride, mode,
        _ptr(critical_counts), _ptr(ambient_head_mask), float(sm_scale), num_splits, _ptr(out), _ptr(out_lse),
        _ptr(workspace), workspace.numel(), _stream(kv.device)))
    return out, out_lse


def sa_sparse_decode_noalloc(kv: PagedKV, q: torch.Tensor, page_lists: torch.Tensor, page_counts: torch.Tensor,
                             *, mode: int, sm_scale: float, critical_counts: Optional[torch.Tensor] = None,
                             ambient_head_mask: Optional[torch.Tensor] = None, num_splits: int = 0,
                             out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
                             want_lse: bool = True):
    """sa_sparse_decode with the split partials in the library's static scratch (no workspace).

    Returns (out, lse).  Outputs the caller does not pass are allocated here by
    torch; the library call itself allocates nothing.
    """
    B, T, Hq, _ = q.shape
    list_stride = page_lists.shape[-1]
    if out is None:
        out = torch.empty((B, T, Hq, kv.d_v), dtype=kv.dtype, device=kv.device)
    if out_lse is None and want_lse:
        out_lse = torch.empty((B, T, Hq), dtype=torch.float32, device=kv.device)
    _check(load_library().sa_sparse_decode_noalloc(
        kv.ref, B, _ptr(q), T, Hq, _ptr(page_lists), _ptr(page_counts), list_stride, mode,
        _ptr(critical_counts), _ptr(ambient_head_mask), float(sm_scale), num_splits, _ptr(out), _ptr(out_lse),
        _stream(kv.device)))
    return out, out_lse


def sa_select_decode(kv: PagedKV, q: torch.Tensor, page_summary: torch.Tensor, *, sink_pages: int,
                     window_pages: int, top_k: int, sm_scale: float, refresh_newest_page: bool = False,
                     list_stride: Optional[int] = None, out=None, want_lse: bool = True):
    """Selection and decode of per-KV-head lists in one call.  Returns (page_lists
    [B][Hkv][list_stride] int32, page_counts [B][Hkv], out [B][T][Hq][d_v], lse or None)."""
    B, T, Hq, _ = q.shape
    if list_stride is None:
        list_stride = max(1, min(kv.max_pages, sink_pages + window_pages + top_k))
    if out is None:
        lists = torch.full((B, kv.n_kv_heads, list_stride), -1, dtype=torch.int32, device=kv.device)
        counts = torch.zeros((B, kv.n_kv_heads), dtype=torch.int32, device=kv.device)
        o = torch.empty((B, T, Hq, kv.d_v), dtype=kv.dtype, device=kv.device)
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=kv.device) if want_lse else None
    else:
        lists, counts, o, lse = out
    _check(load_library().sa_select_decode(
        kv.ref, B, _ptr(q), T, Hq, _ptr(page_summary), 1 if refresh_newest_page else 0, sink_pages, window_pages,
        top_k, _ptr(lists), list_stride, _ptr(counts), float(sm_scale), _ptr(o), _ptr(lse), _stream(kv.device)))
    return lists, counts, o, lse


def sa_block_sparse_prefill_workspace_size(kv: PagedKV, q_len: int, n_q_heads: int, n_kv_blocks: int) -> int:
    return load_library().sa_block_sparse_prefill_workspace_size(kv.ref, q_len, n_q_heads, n_kv_blocks)


def sa_block_sparse_prefill(kv: PagedKV, seq: int, q: torch.Tensor, q_start: int, block_mask: torch.Tensor,
                            block_q: int, sm_scale: float, *, out: Optional[torch.Tensor] = None,
                            out_lse: Optional[torch.Tensor] = None, block_table_out=None, block_counts_out=None,
                            workspace: Optional[torch.Tensor] = None):
    """Returns (out [q_len][Hq][d], lse [q_len][Hq], block_table_out [Hkv][nkb], block_counts_out [Hkv])."""
    q_len, Hq, _ = q.shape
    nkb = block_mask.shape[-1]
    if out is None:
        out = torch.empty((q_len, Hq, kv.d_v), dtype=kv.dtype, device=kv.device)
    if out_lse is None:
        out_lse = torch.empty((q_len, Hq), dtype=torch.float32, device=kv.device)
    if block_table_out is None:
        block_table_out = torch.full((kv.n_kv_heads, nkb), -1, dtype=torch.int32, device=kv.device)
    if block_counts_out is None:
        block_counts_out = torch.zeros((kv.n_kv_heads,), dtype=torch.int32, device=kv.device)
    if workspace is None:
        nbytes = sa_block_sparse_prefill_workspace_size(kv, q_len, Hq, nkb)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=kv.device)
    _check(load_library().sa_block_sparse_prefill(
        kv.ref, seq, _ptr(q), q_len, q_start, Hq, _ptr(block_mask), block_q, nkb, _ptr(block_table_out),
        _ptr(block_counts_out), float(sm_scale), _ptr(out), _ptr(out_lse), _ptr(workspace), workspace.numel(),
        _stream(kv.device)))
    return out, out_lse, block_table_out, block_counts_out


def sa_prefill_block_mask(kv: PagedKV, seq: int, q: torch.Tensor, q_start: int, page_summary: torch.Tensor,
                          block_q: int, sm_scale: float, *, top_k: Optional[int] = None,
                          max_gap: Optional[float] = None, n_kv_blocks: Optional[int] = None,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Returns the uint8 block mask [Hq][ceil(q_len/block_q)][n_kv_blocks]; give exactly one of top_k / max_gap."""
    if (top_k is None) == (max_gap is None):
        raise ValueError("give exactly one of top_k and max_gap")
    q_len, Hq, _ = q.shape
    if n_kv_blocks is None:
        n_kv_blocks = (q_start + q_len + kv.page_size - 1) // kv.page_size
    nqb = (q_len + block_q - 1) // block_q
    if out is None:
        out = torch.empty((Hq, nqb, n_kv_blocks), dtype=torch.uint8, device=kv.device)
    _check(load_library().sa_prefill_block_mask(
        kv.ref, seq, _ptr(q), q_len, q_start, Hq, _ptr(page_summary), block_q, n_kv_blocks, float(sm_scale),
        -1 if top_k is None else int(top_k), float("inf") if max_gap is None else float(max_gap), _ptr(out),
        _stream(kv.device)))
    return out


def sa_page_value_summary(kv: PagedKV, last_pages: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-page mean value rows [n_phys_pages][n_kv_heads][d_v] fp32 (NaN where not written)."""
    if out is None:
        out = torch.full((kv.c.n_phys_pages, kv.n_kv_heads, kv.d_v), float("nan"), dtype=torch.float32,
                         device=kv.device)
    _check(load_library().sa_page_value_summary(kv.ref, kv.batch, last_pages, _ptr(out), _stream(kv.device)))
    return out


def sa_prefill_mean_correction_workspace_size(kv: PagedKV, n_kv_blocks: int) -> int:
    return load_library().sa_prefill_mean_correction_workspace_size(kv.ref, n_kv_blocks)


def sa_prefill_mean_correction(kv: PagedKV, seq: int, q: torch.Tensor, q_start: int, block_table: torch.Tensor,
                               block_counts: torch.Tensor, page_summary: torch.Tensor,
                               value_summary: torch.Tensor, sm_scale: float, out: torch.Tensor,
                               out_lse: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Adds the prefill's skipped causal blocks back as mean terms; rewrites (out, out_lse) in place."""
    q_len, Hq, _ = q.shape
    nkb = block_table.shape[-1]
    if workspace is None:
        nbytes = sa_prefill_mean_correction_workspace_size(kv, nkb)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=kv.device)
    _check(load_library().sa_prefill_mean_correction(
        kv.ref, seq, _ptr(q), q_len, q_start, Hq, _ptr(block_table), _ptr(block_counts), nkb, _ptr(page_summary),
        _ptr(value_summary), float(sm_scale), _ptr(out), _ptr(out_lse), _ptr(workspace), workspace.numel(),
        _stream(kv.device)))
    return out, out_lse


def sa_head_page_mass_workspace_size(kv: PagedKV, q_tokens: int, n_q_heads: int) -> int:
    return load_library().sa_head_page_mass_workspace_size(kv.ref, kv.batch, q_tokens, n_q_heads)


def sa_head_page_mass(kv: PagedKV, q: torch.Tensor, page_summary: torch.Tensor, sm_scale: float, *,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Estimated attention mass [B][Hq][max_pages] fp32 of every (query head, page); q [B][T][Hq][d] bf16."""
    B, T, Hq, _ = q.shape
    if out is None:
        out = torch.full((B, Hq, kv.max_pages), float("nan"), dtype=torch.float32, device=kv.device)
    if workspace is None:
        nbytes = sa_head_page_mass_workspace_size(kv, T, Hq)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=kv.device)
    _check(load_library().sa_head_page_mass(kv.ref, B, _ptr(q), T, Hq, _ptr(page_summary), float(sm_scale),
                                            _ptr(out), _ptr(workspace), workspace.numel(), _stream(kv.device)))
    return out


def sa_autotune_tiers_workspace_size(kv: PagedKV, n_heads: int) -> int:
    return load_library().sa_autotune_tiers_workspace_size(kv.ref, kv.batch, n_heads)


def sa_autotune_tiers(kv: PagedKV, head_mass: torch.Tensor, scores: torch.Tensor, *, q_tokens: int,
                      sink_pages: int, window_pages: int, budget: int, alphas, ambient_heads,
                      workspace: Optional[torch.Tensor] = None, out=None):
    """Returns (coverage [n_alphas][n_heads] fp32, choice int32[3] = alpha index, head index, beta);
    alphas and ambient_heads are host sequences."""
    Hq = head_mass.shape[1]
    na, nh = len(alphas), len(ambient_heads)
    if out is None:
        cov = torch.empty((na, nh), dtype=torch.float32, device=kv.device)
        choice = torch.empty((3,), dtype=torch.int32, device=kv.device)
    else:
        cov, choice = out
    if workspace is None:
        nbytes = sa_autotune_tiers_workspace_size(kv, nh)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=kv.device)
    a = (c_int32 * na)(*[int(x) for x in alphas])
    h = (c_int32 * nh)(*[int(x) for x in ambient_heads])
    _check(load_library().sa_autotune_tiers(
        kv.ref, kv.batch, q_tokens, Hq, _ptr(head_mass), _ptr(scores), scores.shape[-1], sink_pages, window_pages,
        budget, ctypes.cast(a, ctypes.c_void_p), na, ctypes.cast(h, ctypes.c_void_p), nh, _ptr(cov), _ptr(choice),
        _ptr(workspace), workspace.numel(), _stream(kv.device)))
    return cov, choice


def sa_ambient_head_mask(kv: PagedKV, head_mass: torch.Tensor, page_lists: torch.Tensor, page_counts: torch.Tensor,
                         critical_counts: torch.Tensor, ambient_heads: int,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Ambient head mask [B][max_pages][ceil(Hq/32)] int32 words for tiered per-KV-head lists."""
    Hq = head_mass.shape[1]
    if out is None:
        out = torch.empty((kv.batch, kv.max_pages, (Hq + 31) // 32), dtype=torch.int32, device=kv.device)
    _check(load_library().sa_ambient_head_mask(
        kv.ref, kv.batch, Hq, _ptr(head_mass), _ptr(page_lists), page_lists.shape[-1], _ptr(page_counts),
        _ptr(critical_counts), int(ambient_heads), _ptr(out), _stream(kv.device)))
    return out


def sa_set_debug_validate(on: bool) -> bool:
    """Turn the library's device-side data checks on or off; returns the previous setting."""
    return bool(load_library().sa_set_debug_validate(1 if on else 0))


def sa_version() -> int:
    return load_library().sa_version()
