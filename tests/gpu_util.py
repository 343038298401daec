"""Helpers for the GPU parity tests: upload a seeded workload, placed by the oracle,
call the library through its C ABI, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import paged_kv_cache_pg_amd as P
from paged_kv_cache_pg_amd.inputs import Workload

DT = {"bf16": P.PAGED_BF16, "f32": P.PAGED_F32}
TOL = 2e-3  # max over a row of |x - ref| / max over the row of |ref|


def dev(a: np.ndarray) -> torch.Tensor:
    """Upload a numpy array byte for byte (uint16 bf16 bits travel as int16)."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bytes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


class Placed:
    """A workload placed in one arena (paged, through its table) or contiguously (no table)."""

    def __init__(self, w: Workload, paged: bool = True, guard: int = 4096, table=None, cap=None):
        self.w = w
        self.paged = paged
        cap = max(w.lens + [1]) if cap is None else cap  # positions a contiguous stream holds
        self.page_pos = w.page_pos if paged else cap
        self.table_np = (w.table if table is None else table) if paged else None
        self.olay = O.PageLayout(w.n_kv_heads, w.head_dim, self.page_pos, w.dtype, idx_dim=w.idx_dim)
        self.lay = P.ArenaLayout(w.n_kv_heads, w.head_dim, self.page_pos, DT[w.dtype], idx_dim=w.idx_dim)
        n_pages = w.n_pages if paged else w.n_streams
        arena = O.place(self.olay, self.table_np, n_pages, w.lens, w.K, w.V, w.IK)
        self.guard = guard
        self.buf = dev(np.concatenate([np.full(guard, 0xA5, np.uint8), arena, np.full(guard, 0xA5, np.uint8)]))
        self.arena_np = arena
        self.base = self.buf.data_ptr() + guard
        self.table = dev(self.table_np.astype(np.int32)) if self.table_np is not None else None
        self.pg = P.make_pg(self.table, self.page_pos, self.lay.page_elems)
        self.kv = P.make_kv(self.base + self.lay.k_off, self.base + self.lay.v_off, DT[w.dtype], w.n_kv_heads,
                            w.head_dim)
        self.lens = dev(np.array(w.lens, np.int32))

    @property
    def ik(self) -> int:
        return self.base + self.lay.ik_off

    @property
    def pooled(self) -> int:
        return self.base + self.lay.pool_off

    def arena_now(self) -> np.ndarray:
        b = host_bytes(self.buf)
        return b[self.guard:len(b) - self.guard]

    def guards_intact(self) -> bool:
        b = host_bytes(self.buf)
        return bool(np.all(b[:self.guard] == 0xA5) and np.all(b[len(b) - self.guard:] == 0xA5))


def guarded_out(shape, guard_floats: int = 1024):
    """An fp32 output with canary bands on both sides: returns (full buffer, view)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * guard_floats,), float("nan"), dtype=torch.float32, device="cuda")
    buf.view(torch.int32)[:guard_floats] = 0x5A5A5A5A
    buf.view(torch.int32)[guard_floats + n:] = 0x5A5A5A5A
    return buf, buf[guard_floats:guard_floats + n].view(*shape)


def out_guards_intact(buf, guard_floats: int = 1024) -> bool:
    v = buf.view(torch.int32).cpu().numpy()
    return bool(np.all(v[:guard_floats] == 0x5A5A5A5A) and np.all(v[-guard_floats:] == 0x5A5A5A5A))


def decode(pl: Placed, q: torch.Tensor, scale: float, lens=None, max_len=None, out=None):
    w = pl.w
    S = w.n_streams
    max_len = max_len if max_len is not None else max(w.lens + [0])
    ws_bytes = P.paged_attn_decode_workspace(S, w.n_q_heads, max_len)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    if out is None:
        out = torch.empty((S, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    P.paged_attn_decode(q, DT[w.dtype], w.n_q_heads, pl.kv, pl.pg, pl.lens if lens is None else lens, S, max_len,
                        scale, out, ws)
    return out


def rel_err_rows(x: np.ndarray, ref: np.ndarray) -> float:
    """Worst row of max|x - ref| / max|ref| over the last axis."""
    x = x.reshape(-1, x.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.max(np.abs(x - r), axis=1)
    den = np.max(np.abs(r), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if len(num) else 0.0


class PlacedFp8:
    """e4m3 rows and their scales placed by the oracle in one arena (paged through a table, or contiguously)."""

    def __init__(self, lens, n_kv_heads, page_pos, KC, VC, KS, VS, table=None, n_pages=None, guard: int = 4096):
        self.lens_list = [int(x) for x in lens]
        cap = max(self.lens_list + [1])
        self.paged = table is not None
        self.page_pos = page_pos if self.paged else max(cap, KC.shape[2])
        self.table_np = table
        self.olay = O.PageLayout(n_kv_heads, 256, self.page_pos, "fp8")
        self.lay = P.ArenaLayout(n_kv_heads, 256, self.page_pos, P.PAGED_FP8_E4M3)
        assert self.lay.page_bytes == self.olay.page_bytes and self.lay.ks_off == self.olay.ks_off
        n_pages = n_pages if self.paged else len(self.lens_list)
        arena = O.place_fp8(self.olay, table, n_pages, self.lens_list, KC, VC, KS, VS)
        self.arena_np = arena
        self.guard = guard
        self.buf = dev(np.concatenate([np.full(guard, 0xA5, np.uint8), arena, np.full(guard, 0xA5, np.uint8)]))
        self.base = self.buf.data_ptr() + guard
        self.table = dev(table.astype(np.int32)) if self.paged else None
        self.pg = P.make_pg(self.table, self.page_pos, self.lay.page_elems)
        self.kv = P.make_kv(self.base + self.lay.k_off, self.base + self.lay.v_off, P.PAGED_FP8_E4M3, n_kv_heads,
                            256, self.base + self.lay.ks_off, self.base + self.lay.vs_off)
        self.lens = dev(np.array(self.lens_list, np.int32))

    def arena_now(self) -> np.ndarray:
        b = host_bytes(self.buf)
        return b[self.guard:len(b) - self.guard]

    def guards_intact(self) -> bool:
        b = host_bytes(self.buf)
        return bool(np.all(b[:self.guard] == 0xA5) and np.all(b[len(b) - self.guard:] == 0xA5))


def decode_fp8(pl: PlacedFp8, q: torch.Tensor, n_q_heads: int, scale: float, max_len=None, out=None):
    S = len(pl.lens_list)
    max_len = max_len if max_len is not None else max(pl.lens_list + [0])
    ws_bytes = P.paged_attn_decode_workspace(S, n_q_heads, max_len)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    if out is None:
        out = torch.empty((S, n_q_heads, 256), dtype=torch.float32, device="cuda")
    P.paged_attn_decode(q, P.PAGED_BF16, n_q_heads, pl.kv, pl.pg, pl.lens, S, max_len, scale, out, ws)
    return out
