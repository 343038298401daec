"""Arena layout of one attention layer inside a page (the library side's own description).

TensorFold PR #1169 "What this changes": each page covers n positions and stores,
per attention layer, their keys, values and indexer keys plus one pooled row for
each of their n/4 blocks; each cache pointer addresses its layer's share of page 0.
PR #1170 commit 3f5b87d gives the in-page order [key, value][head][position][row].
This package lays a page out as

    K [Hkv][n][D] | V [Hkv][n][D] | IK [n][DI] | POOL [n/4][DI] float32

and hands the kernels one base pointer per region.  e4m3 pages (PR #1170 commit
5c09685: fp8 rows keep e4m3 codes plus a float32 scale, and page sizes count bytes) hold

    K codes [Hkv][n][D] | V codes [Hkv][n][D] | K scales [Hkv][n] float32 | V scales [Hkv][n] float32

padded to 16 bytes, with no indexer keys.
"""
from __future__ import annotations

from dataclasses import dataclass

from .binding import ESIZE, PAGED_FP8_E4M3


@dataclass(frozen=True)
class ArenaLayout:
    n_kv_heads: int
    head_dim: int
    page_pos: int
    dtype: int            # PAGED_F32, PAGED_BF16 or PAGED_FP8_E4M3
    idx_dim: int = 0

    @property
    def esize(self) -> int:
        return ESIZE[self.dtype]

    @property
    def kv_bytes(self) -> int:
        return self.n_kv_heads * self.page_pos * self.head_dim * self.esize

    @property
    def k_off(self) -> int:
        return 0

    @property
    def v_off(self) -> int:
        return self.kv_bytes

    @property
    def ik_off(self) -> int:
        return 2 * self.kv_bytes

    @property
    def scale_bytes(self) -> int:
        return self.n_kv_heads * self.page_pos * 4

    @property
    def ks_off(self) -> int:
        return 2 * self.kv_bytes

    @property
    def vs_off(self) -> int:
        return 2 * self.kv_bytes + self.scale_bytes

    @property
    def pool_off(self) -> int:
        return self.ik_off + self.page_pos * self.idx_dim * self.esize

    @property
    def page_bytes(self) -> int:
        if self.dtype == PAGED_FP8_E4M3:
            assert not self.idx_dim, "e4m3 pages hold no indexer keys"
            return (2 * self.kv_bytes + 2 * self.scale_bytes + 15) // 16 * 16
        if not self.idx_dim:
            return 2 * self.kv_bytes
        return self.pool_off + (self.page_pos // 4) * self.idx_dim * 4

    @property
    def page_elems(self) -> int:
        return self.page_bytes // self.esize
