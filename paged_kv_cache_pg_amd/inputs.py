"""Seeded synthetic inputs for paged KV-cache attention.

This module is the only code that the CPU oracle's tests and the HIP path share.
It draws random tensors and page tables and holds none of the method's
arithmetic: no row addressing, no attention, no pooling, no scoring.

Recipe (the same for every workload):
  * generator: ``numpy.random.default_rng(seed)``;
  * draw order: q, K, V, IK (indexer keys), qI (indexer queries), then the
    page-table permutation;
  * values are N(0, 1) drawn in float32; where a workload is bf16 each draw is
    rounded to the nearest bf16 (ties to even) and both sides read those bits.

Page tables come in the three shapes the pages test with (PR #1169 "What this
changes" and "Receipt"; PR #1170 commit 85aeb4b):
  * ``"reversed"`` -- logical page i of a stream sits at arena page P-1-i;
  * ``"shuffled"`` -- one seeded permutation of all streams' pages in one arena;
  * ``None``       -- no table: each stream's rows are contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "draw_e4m3_codes",
    "draw_row_scales",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "Workload",
    "make_workload",
    "make_table",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs only: u + 0x8000 never wraps below the NaN patterns
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the float32 values they encode (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, shape, dtype: str):
    """N(0,1) in float32, rounded to bf16 bits when dtype == 'bf16'."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def draw_e4m3_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform e4m3 codes (uint8) over the 254 codes that are not NaN (0x7F and 0xFF excluded),
    so every magnitude from the subnormals to 448 and both signs appear."""
    i = rng.integers(0, 254, size=shape, dtype=np.int64)
    return (i + (i >= 0x7F)).astype(np.uint8)


def draw_row_scales(rng: np.random.Generator, shape, lo: float = 2.0 ** -8, hi: float = 2.0 ** -5) -> np.ndarray:
    """Positive float32 row scales, log-uniform in [lo, hi)."""
    return np.exp2(rng.uniform(np.log2(lo), np.log2(hi), size=shape)).astype(np.float32)


def make_table(kind: Optional[str], pages_per_stream: Sequence[int], rng: Optional[np.random.Generator] = None,
               stride: Optional[int] = None):
    """Return (table [S][stride] int32 or None, number of arena pages).

    Entries past a stream's own pages are filled with 0 (a valid page) and are never read.
    """
    S = len(pages_per_stream)
    total = int(sum(pages_per_stream))
    if kind is None:
        return None, S
    stride = int(stride if stride is not None else max(1, max(pages_per_stream)))
    table = np.zeros((S, stride), dtype=np.int32)
    if kind == "reversed":
        base = 0
        for s, n in enumerate(pages_per_stream):
            for i in range(n):
                table[s, i] = base + (n - 1 - i)
            base += n
    elif kind == "shuffled":
        if rng is None:
            raise ValueError("a shuffled table needs the workload's generator")
        perm = rng.permutation(total).astype(np.int32)
        base = 0
        for s, n in enumerate(pages_per_stream):
            table[s, :n] = perm[base:base + n]
            base += n
    elif kind == "identity":
        base = 0
        for s, n in enumerate(pages_per_stream):
            table[s, :n] = np.arange(base, base + n, dtype=np.int32)
            base += n
    else:
        raise ValueError(f"unknown table kind {kind!r}")
    return table, total


@dataclass
class Workload:
    """Logical (contiguous) tensors of one synthetic workload, plus its page table.

    Element arrays hold bf16 bit patterns (uint16) for bf16 workloads and float32
    values for f32 workloads.  Shapes:
      q   [S][Hq][D]            decode queries (or [Nq][Hq][D] for a prefill chunk)
      K,V [S][Hkv][Lmax][D]     cached keys / values, row p of stream s valid for p < lens[s]
      IK  [S][Lmax][DI]         indexer keys (optional)
      qI  [S][Hi][DI]           indexer queries (optional)
    """
    dtype: str
    lens: List[int]
    page_pos: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    IK: Optional[np.ndarray] = None
    qI: Optional[np.ndarray] = None
    table: Optional[np.ndarray] = None
    n_pages: int = 0
    table_kind: Optional[str] = None
    idx_dim: int = 0
    n_idx_heads: int = 0
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def n_streams(self) -> int:
        return len(self.lens)

    @property
    def max_len(self) -> int:
        return int(max(self.lens)) if self.lens else 0

    def as_f64(self, name: str) -> np.ndarray:
        """A tensor's exact values widened to float64."""
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def make_workload(seed: int, lens: Sequence[int], page_pos: int, n_q_heads: int, n_kv_heads: int,
                  head_dim: int = 256, dtype: str = "bf16", table_kind: Optional[str] = "shuffled",
                  n_queries: Optional[int] = None, idx_dim: int = 0, n_idx_heads: int = 0,
                  q_dtype: Optional[str] = None, cap: Optional[int] = None) -> Workload:
    """Draw one workload in the fixed order q, K, V, IK, qI, table.

    ``n_queries`` switches q to a prefill chunk [n_queries][Hq][D] (one stream).
    ``cap`` is the row capacity per stream of the logical tensors (default: max(lens)).
    """
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    S = len(lens)
    lmax = int(cap if cap is not None else max(lens + [1]))
    qd = q_dtype or dtype
    if n_queries is None:
        q = _draw(rng, (S, n_q_heads, head_dim), qd)
    else:
        q = _draw(rng, (int(n_queries), n_q_heads, head_dim), qd)
    K = _draw(rng, (S, n_kv_heads, lmax, head_dim), dtype)
    V = _draw(rng, (S, n_kv_heads, lmax, head_dim), dtype)
    IK = _draw(rng, (S, lmax, idx_dim), dtype) if idx_dim else None
    qI = _draw(rng, (S, n_idx_heads, idx_dim), qd) if idx_dim else None
    pages = [(l + page_pos - 1) // page_pos for l in lens]
    pages = [max(1, p) for p in pages]
    table, n_pages = make_table(table_kind, pages, rng)
    return Workload(dtype=dtype, lens=lens, page_pos=page_pos, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                    head_dim=head_dim, q=q, K=K, V=V, IK=IK, qI=qI, table=table, n_pages=n_pages,
                    table_kind=table_kind, idx_dim=idx_dim, n_idx_heads=n_idx_heads, seed=seed)
