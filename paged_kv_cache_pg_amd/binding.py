"""Thin ctypes binding over libpagedattn.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
computation of its own: tensors become device pointers, the current PyTorch
stream becomes the hipStream_t, a negative status becomes a PagedError.  The
library must be built (``python -m paged_kv_cache_pg_amd.build``); there is no
other path: a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_float, c_int32, c_int64, c_size_t, c_void_p, POINTER
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PAGED_F32 = 0
PAGED_BF16 = 1
PAGED_FP8_E4M3 = 2
DTYPES = {"f32": PAGED_F32, "bf16": PAGED_BF16, "fp8": PAGED_FP8_E4M3}
ESIZE = {PAGED_F32: 4, PAGED_BF16: 2, PAGED_FP8_E4M3: 1}

PAGED_OK = 0
PAGED_EINVAL = -1
PAGED_EUNSUPPORTED = -2
PAGED_EWORKSPACE = -3
PAGED_EHIP = -4
PAGED_EFULL = -5
PAGED_ESCRATCH = -6
NOALLOC_SCRATCH_BYTES = 1024 * 16 * (256 + 2) * 4  # PAGED_NOALLOC_SCRATCH_BYTES


class PagedError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


class PgStruct(ctypes.Structure):
    _fields_ = [("table", c_void_p), ("table_stride", c_int32), ("page_pos", c_int32),
                ("page_elems", c_int64), ("reserved", c_int64)]


class KvStruct(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("dtype", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("reserved", c_int32), ("k_scale", c_void_p), ("v_scale", c_void_p)]


_lib = None

_SIGS = {
    "paged_attn_decode": (c_int32, [c_void_p, c_int32, c_int32, POINTER(KvStruct), POINTER(PgStruct), c_void_p,
                                    c_int32, c_int32, c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "paged_attn_decode_workspace": (c_size_t, [c_int32, c_int32, c_int32]),
    "paged_attn_decode_noalloc": (c_int32, [c_void_p, c_int32, c_int32, POINTER(KvStruct), POINTER(PgStruct),
                                            c_void_p, c_int32, c_int32, c_float, c_void_p, c_void_p]),
    "paged_attn_decode_window": (c_int32, [c_void_p, c_int32, c_int32, c_int32, POINTER(KvStruct),
                                           POINTER(PgStruct), c_void_p, c_int32, c_int32, c_float, c_void_p,
                                           c_void_p, c_size_t, c_void_p]),
    "paged_attn_decode_window_workspace": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "paged_attn_prefill": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, POINTER(KvStruct),
                                     POINTER(PgStruct), c_int32, c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "paged_attn_prefill_workspace": (c_size_t, [c_int32, c_int32, c_int32]),
    "paged_pool_blocks": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, POINTER(PgStruct), c_void_p, c_void_p,
                                    c_int32, c_int32, c_void_p]),
    "paged_block_scores_topk": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_int32, POINTER(PgStruct),
                                          c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_size_t, c_void_p]),
    "paged_topk_workspace": (c_size_t, [c_int32, c_int32, c_int32]),
    "paged_sparse_attn": (c_int32, [c_void_p, c_int32, c_int32, POINTER(KvStruct), POINTER(PgStruct), c_void_p,
                                    c_void_p, c_int32, c_int32, c_int32, c_float, c_void_p, c_void_p, c_size_t,
                                    c_void_p]),
    "paged_sparse_attn_workspace": (c_size_t, [c_int32, c_int32, c_int32]),
    "paged_rows_store": (c_int32, [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int32, c_int32, c_int32,
                                   POINTER(PgStruct), c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
    "paged_rows_gather": (c_int32, [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int32, c_int32, c_int32,
                                    POINTER(PgStruct), c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
    "paged_row_offsets": (c_int32, [POINTER(PgStruct), c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_int32, c_void_p]),
    "paged_strerror": (ctypes.c_char_p, [c_int32]),
    "paged_kv_append": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, POINTER(KvStruct), c_void_p, c_void_p,
                                  c_int32, POINTER(PgStruct), c_void_p, c_int32, c_int32, c_void_p]),
    "paged_pool_state_bytes": (c_size_t, [c_int32]),
    "paged_pool_init": (c_int32, [c_void_p, c_size_t, c_int32]),
    "paged_pool_alloc": (c_int32, [c_void_p, c_int32, c_void_p]),
    "paged_pool_free": (c_int32, [c_void_p, c_void_p, c_int32]),
    "paged_pool_claim_run": (c_int32, [c_void_p, c_int32, c_void_p]),
    "paged_pool_release_run": (c_int32, [c_void_p, c_int32, c_int32]),
    "paged_pool_free_count": (c_int32, [c_void_p]),
}


def lib():
    """Load libpagedattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m paged_kv_cache_pg_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().paged_strerror(status).decode()


def _p(x) -> int:
    """Device (or host) address of a tensor, an int address, or 0 for None."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != PAGED_OK:
        raise PagedError(status, where)


def make_pg(table, page_pos: int, page_elems: int, table_stride: Optional[int] = None) -> PgStruct:
    """The pages' Pg argument: a table (device int32 tensor [S][stride] or None), positions and elements a page."""
    if table is not None and table_stride is None:
        table_stride = int(table.shape[-1])
    pg = PgStruct(_p(table), int(table_stride or 0), int(page_pos), int(page_elems), 0)
    pg._keep = table  # a tensor passed here stays allocated while the struct lives
    return pg


def make_kv(k, v, dtype: int, n_kv_heads: int, head_dim: int = 256, k_scale=None, v_scale=None) -> KvStruct:
    """K and V region bases (tensors or int device addresses) of one layer; for PAGED_FP8_E4M3 also the
    K and V scale region bases."""
    kv = KvStruct(_p(k), _p(v), int(dtype), int(n_kv_heads), int(head_dim), 0, _p(k_scale), _p(v_scale))
    kv._keep = (k, v, k_scale, v_scale)  # tensors passed here stay allocated while the struct lives
    return kv


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def paged_attn_decode_workspace(n_streams: int, n_q_heads: int, max_len: int) -> int:
    return int(lib().paged_attn_decode_workspace(n_streams, n_q_heads, max_len))


def paged_attn_decode(q, q_dtype: int, n_q_heads: int, kv: KvStruct, pg: PgStruct, seq_lens, n_streams: int,
                      max_len: int, scale: float, out, workspace, workspace_bytes: Optional[int] = None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None and workspace is not None else (workspace_bytes or 0)
    _check(lib().paged_attn_decode(_p(q), q_dtype, n_q_heads, ctypes.byref(kv), ctypes.byref(pg), _p(seq_lens),
                                   n_streams, max_len, scale, _p(out), _p(workspace), wb, _stream(stream)),
           "paged_attn_decode")


def paged_attn_decode_noalloc(q, q_dtype: int, n_q_heads: int, kv: KvStruct, pg: PgStruct, seq_lens, n_streams: int,
                              max_len: int, scale: float, out, stream=None):
    _check(lib().paged_attn_decode_noalloc(_p(q), q_dtype, n_q_heads, ctypes.byref(kv), ctypes.byref(pg),
                                           _p(seq_lens), n_streams, max_len, scale, _p(out), _stream(stream)),
           "paged_attn_decode_noalloc")


def paged_attn_decode_window_workspace(n_streams: int, n_q_heads: int, n_window: int, max_len: int) -> int:
    return int(lib().paged_attn_decode_window_workspace(n_streams, n_q_heads, n_window, max_len))


def paged_attn_decode_window(q, q_dtype: int, n_q_heads: int, n_window: int, kv: KvStruct, pg: PgStruct, seq_lens,
                             n_streams: int, max_len: int, scale: float, out, workspace,
                             workspace_bytes: Optional[int] = None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None and workspace is not None else (workspace_bytes or 0)
    _check(lib().paged_attn_decode_window(_p(q), q_dtype, n_q_heads, n_window, ctypes.byref(kv), ctypes.byref(pg),
                                          _p(seq_lens), n_streams, max_len, scale, _p(out), _p(workspace), wb,
                                          _stream(stream)),
           "paged_attn_decode_window")


def paged_attn_prefill_workspace(n_q: int, n_q_heads: int, kv_len: int) -> int:
    return int(lib().paged_attn_prefill_workspace(n_q, n_q_heads, kv_len))


def paged_attn_prefill(q, q_dtype: int, n_q: int, q_pos0: int, n_q_heads: int, kv: KvStruct, pg: PgStruct,
                       causal: bool, scale: float, out, workspace=None, workspace_bytes: Optional[int] = None,
                       stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None and workspace is not None else (workspace_bytes or 0)
    _check(lib().paged_attn_prefill(_p(q), q_dtype, n_q, q_pos0, n_q_heads, ctypes.byref(kv), ctypes.byref(pg),
                                    int(bool(causal)), scale, _p(out), _p(workspace), wb, _stream(stream)),
           "paged_attn_prefill")


def paged_pool_blocks(ik, pooled, idx_dim: int, arena_dtype: int, pg: PgStruct, block_begin, block_end,
                      n_streams: int, max_len: int, stream=None):
    _check(lib().paged_pool_blocks(_p(ik), _p(pooled), idx_dim, arena_dtype, ctypes.byref(pg), _p(block_begin),
                                   _p(block_end), n_streams, max_len, _stream(stream)), "paged_pool_blocks")


def paged_topk_workspace(n_streams: int, max_len: int, k: int) -> int:
    return int(lib().paged_topk_workspace(n_streams, max_len, k))


def paged_block_scores_topk(qi, qi_dtype: int, n_idx_heads: int, idx_dim: int, pooled, arena_dtype: int,
                            pg: PgStruct, seq_lens, n_streams: int, max_len: int, k: int, out_ids, out_count,
                            out_scores, workspace, workspace_bytes: Optional[int] = None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None and workspace is not None else (workspace_bytes or 0)
    _check(lib().paged_block_scores_topk(_p(qi), qi_dtype, n_idx_heads, idx_dim, _p(pooled), arena_dtype,
                                         ctypes.byref(pg), _p(seq_lens), n_streams, max_len, k, _p(out_ids),
                                         _p(out_count), _p(out_scores), _p(workspace), wb, _stream(stream)),
           "paged_block_scores_topk")


def paged_sparse_attn_workspace(n_streams: int, n_q_heads: int, k: int) -> int:
    return int(lib().paged_sparse_attn_workspace(n_streams, n_q_heads, k))


def paged_sparse_attn(q, q_dtype: int, n_q_heads: int, kv: KvStruct, pg: PgStruct, block_ids, n_selected, k: int,
                      n_streams: int, max_len: int, scale: float, out, workspace,
                      workspace_bytes: Optional[int] = None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None and workspace is not None else (workspace_bytes or 0)
    _check(lib().paged_sparse_attn(_p(q), q_dtype, n_q_heads, ctypes.byref(kv), ctypes.byref(pg), _p(block_ids),
                                   _p(n_selected), k, n_streams, max_len, scale, _p(out), _p(workspace), wb,
                                   _stream(stream)), "paged_sparse_attn")


def paged_rows_store(src, stride_s: int, stride_h: int, stride_p: int, region, n_heads: int, row_elems: int,
                     dtype: int, pg: PgStruct, pos_begin, pos_end, n_streams: int, max_len: int, stream=None):
    _check(lib().paged_rows_store(_p(src), stride_s, stride_h, stride_p, _p(region), n_heads, row_elems, dtype,
                                  ctypes.byref(pg), _p(pos_begin), _p(pos_end), n_streams, max_len,
                                  _stream(stream)), "paged_rows_store")


def paged_rows_gather(dst, stride_s: int, stride_h: int, stride_p: int, region, n_heads: int, row_elems: int,
                      dtype: int, pg: PgStruct, pos_begin, pos_end, n_streams: int, max_len: int, stream=None):
    _check(lib().paged_rows_gather(_p(dst), stride_s, stride_h, stride_p, _p(region), n_heads, row_elems, dtype,
                                   ctypes.byref(pg), _p(pos_begin), _p(pos_end), n_streams, max_len,
                                   _stream(stream)), "paged_rows_gather")


def paged_row_offsets(pg: PgStruct, n_streams: int, row_width: int, streams, heads, positions, out, n: int,
                      stream=None):
    _check(lib().paged_row_offsets(ctypes.byref(pg), n_streams, row_width, _p(streams), _p(heads), _p(positions),
                                   _p(out), n, _stream(stream)), "paged_row_offsets")


def paged_kv_append(k_new, v_new, ik_new, n_new: int, kv: KvStruct, ik, pooled, idx_dim: int, pg: PgStruct, pos0,
                    n_streams: int, max_len: int, stream=None):
    _check(lib().paged_kv_append(_p(k_new), _p(v_new), _p(ik_new), n_new, ctypes.byref(kv), _p(ik), _p(pooled),
                                 idx_dim, ctypes.byref(pg), _p(pos0), n_streams, max_len, _stream(stream)),
           "paged_kv_append")


# ---------------------------------------------------------------------------
# Host page pool (state in a caller-owned host buffer, e.g. a numpy uint8 array)
# ---------------------------------------------------------------------------

def _host(a) -> int:
    """Address of a host numpy array (or an int address)."""
    if isinstance(a, int):
        return a
    return a.ctypes.data


def paged_pool_state_bytes(n_pages: int) -> int:
    return int(lib().paged_pool_state_bytes(n_pages))


def paged_pool_init(state, n_pages: int) -> None:
    _check(lib().paged_pool_init(_host(state), state.nbytes, n_pages), "paged_pool_init")


def paged_pool_alloc(state, n: int, pages) -> int:
    """Pages into the int32 array `pages`; returns the status (PAGED_EFULL: nothing taken)."""
    st = int(lib().paged_pool_alloc(_host(state), n, _host(pages)))
    if st not in (PAGED_OK, PAGED_EFULL):
        _check(st, "paged_pool_alloc")
    return st


def paged_pool_free(state, pages, n: int) -> None:
    _check(lib().paged_pool_free(_host(state), _host(pages), n), "paged_pool_free")


def paged_pool_claim_run(state, k: int) -> int:
    """First page of the claimed run, or PAGED_EFULL when no run of k free pages exists."""
    first = ctypes.c_int32(-1)
    st = int(lib().paged_pool_claim_run(_host(state), k, ctypes.addressof(first)))
    if st == PAGED_EFULL:
        return st
    _check(st, "paged_pool_claim_run")
    return int(first.value)


def paged_pool_release_run(state, first: int, k: int) -> None:
    _check(lib().paged_pool_release_run(_host(state), first, k), "paged_pool_release_run")


def paged_pool_free_count(state) -> int:
    n = int(lib().paged_pool_free_count(_host(state)))
    if n < 0:
        _check(n, "paged_pool_free_count")
    return n
