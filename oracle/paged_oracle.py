"""Plain float64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` (its host timing and its spot checks of sampled rows, both
off with ``--no-cpu-baseline``) use it.  It shares no code with the HIP library (its own row
addressing, its own arena layout, its own arithmetic) and is deliberately slow
and obvious.

Sources (page titles and sections; the pages print no source code and no
numeric worked example for these kernels):
  [P1] TensorFold PR #1169, "Flash Next attention caches readable through a
       page table" -- sections "What this changes" and "Receipt".
  [P2] TensorFold PR #1170, "Flash Next CUDA: the streams beside the first take
       KV pages from the core pool" -- description and commit messages 3f5b87d
       (Seg / kv_row), ce5b78d (attention partials) and 85aeb4b (Pg / pg_at).

Where the pages are silent, each function below states the reading it takes.

Parity status per function:
  page_layout / row_offset / place / gather : pinned (hand-derived offsets,
      round trip, red controls)
  decode / prefill / sparse                 : pinned (closed forms, invariants,
      50-digit brute force on tiny shapes)
  decode_window                             : pinned (closed form, equality with the
      causal prefill and with decode, 50-digit brute force)
  pool                                      : pinned (closed forms, exact quarters)
  scores                                    : pinned (exact integer scores,
      one-hot rows, linearity)
  topk                                      : pinned (brute-force sort, ties)
  e4m3_value / e4m3_encode                  : pinned (hand-derived codes, torch's
      float8_e4m3fn conversion, exhaustive round trip, ties, saturation)
  e4m3_quantize_rows / dequantize           : pinned (amax code is +-448, error
      bound of half a code step, zero rows, scale exactness)
  place_fp8 / gather_fp8                    : pinned (hand-derived scale offsets,
      round trip)
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

ESIZE = {"bf16": 2, "f32": 4, "fp8": 1}


# ---------------------------------------------------------------------------
# Row addressing and the page layout
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class PageLayout:
    """Where each region of one attention layer sits inside a page.

    [P1 "What this changes"]: each page covers n positions; per attention layer
    it stores their keys, values and indexer keys, plus one pooled row for each
    of their n/4 blocks.  [P2 commit 3f5b87d]: inside a page the order is
    [key, value][head][position][row].  Reading taken: K [Hkv][n][D], then
    V [Hkv][n][D], then IK [n][DI], then POOL [n/4][DI] float32.
    All offsets are in bytes.

    dtype "fp8" ([P2 commit 5c09685]: a row is e4m3 codes plus an fp32 scale,
    the page size counted in bytes): K codes [Hkv][n][D] bytes, V codes, then
    the K scales [Hkv][n] float32 and the V scales, the page padded to 16 bytes;
    no indexer keys.  Reading taken: the scales sit after the codes in the same
    page, one float32 a row, in the rows' [head][position] order.
    """
    n_kv_heads: int
    head_dim: int
    page_pos: int
    dtype: str
    idx_dim: int = 0

    @property
    def esize(self) -> int:
        return ESIZE[self.dtype]

    @property
    def k_off(self) -> int:
        return 0

    @property
    def v_off(self) -> int:
        return self.n_kv_heads * self.page_pos * self.head_dim * self.esize

    @property
    def ik_off(self) -> int:
        return 2 * self.v_off

    @property
    def ks_off(self) -> int:
        assert self.dtype == "fp8"
        return 2 * self.v_off

    @property
    def vs_off(self) -> int:
        return self.ks_off + self.n_kv_heads * self.page_pos * 4

    @property
    def pool_off(self) -> int:
        return self.ik_off + self.page_pos * self.idx_dim * self.esize

    @property
    def page_bytes(self) -> int:
        if self.dtype == "fp8":
            assert self.idx_dim == 0
            end = self.vs_off + self.n_kv_heads * self.page_pos * 4
            return (end + 15) // 16 * 16
        if self.idx_dim == 0:
            return self.ik_off
        return self.pool_off + (self.page_pos // 4) * self.idx_dim * 4

    @property
    def page_elems(self) -> int:
        """Elements of the arena type in one page (the pages' "elements in a page")."""
        assert self.page_bytes % self.esize == 0
        return self.page_bytes // self.esize


def row_offset(table, page_pos: int, page_elems: int, s: int, h: int, p: int, width: int,
               rows_per_head: Optional[int] = None) -> int:
    """Element offset of row (stream s, head h, position p) in a region whose page part is
    [H][rows_per_head][width].

    [P1 "What this changes"]: without a table the earlier contiguous formula;
    with one, the base of the page containing the position plus the row's offset
    within it.  [P2 commit 3f5b87d]: without a table each stream reserves cap rows
    per head, which is this same expression with page_pos = cap and the implicit table [s].
    """
    if rows_per_head is None:
        rows_per_head = page_pos
    if table is None:
        page = s
        within = p
    else:
        page = int(table[s][p // page_pos])
        within = p % page_pos
    return page * page_elems + (h * rows_per_head + within) * width


def pool_row_offset(table, page_pos: int, page_elems_f32: int, s: int, b: int, width: int) -> int:
    """Float32-element offset of the pooled row of block b (positions 4b..4b+3).

    The block's rows share one page because page_pos is a multiple of 4
    ([P2 "What this changes"]: the positions a page holds must divide by 4); its pooled row is
    row (4b mod n)/4 of that page's POOL region.
    """
    p = 4 * b
    if table is None:
        page, within = s, p
    else:
        page, within = int(table[s][p // page_pos]), p % page_pos
    return page * page_elems_f32 + (within // 4) * width


def place(layout: PageLayout, table, n_pages: int, lens: Sequence[int], K, V, IK=None) -> np.ndarray:
    """Write each stream's rows into a fresh arena (bytes) through the table.

    K, V: [S][Hkv][cap][D] element arrays (uint16 bf16 bits or float32).
    IK:   [S][cap][DI] or None.  Rows past lens[s] are not written.
    The arena starts zero-filled.
    """
    arena = np.zeros(n_pages * layout.page_bytes, dtype=np.uint8)
    es = layout.esize
    D = layout.head_dim
    pe = layout.page_elems
    kview = arena.view(np.uint16 if es == 2 else np.float32)
    for s, L in enumerate(lens):
        # a logical page's rows are consecutive inside its arena page, so copy a page part at once
        for p0 in range(0, L, layout.page_pos):
            n = min(layout.page_pos, L - p0)
            for h in range(layout.n_kv_heads):
                ko = row_offset(table, layout.page_pos, pe, s, h, p0, D) + layout.k_off // es
                vo = row_offset(table, layout.page_pos, pe, s, h, p0, D) + layout.v_off // es
                kview[ko:ko + n * D] = np.asarray(K[s, h, p0:p0 + n]).reshape(-1)
                kview[vo:vo + n * D] = np.asarray(V[s, h, p0:p0 + n]).reshape(-1)
            if IK is not None and layout.idx_dim:
                DI = layout.idx_dim
                io = row_offset(table, layout.page_pos, pe, s, 0, p0, DI) + layout.ik_off // es
                kview[io:io + n * DI] = np.asarray(IK[s, p0:p0 + n]).reshape(-1)
    return arena


def gather(layout: PageLayout, table, arena: np.ndarray, lens: Sequence[int], cap: Optional[int] = None):
    """Inverse of place(): read K, V (and IK when the layout has it) back into logical form,
    one row at a time through row_offset()."""
    es = layout.esize
    D = layout.head_dim
    pe = layout.page_elems
    view = arena.view(np.uint16 if es == 2 else np.float32)
    cap = int(cap if cap is not None else max(list(lens) + [1]))
    S = len(lens)
    K = np.zeros((S, layout.n_kv_heads, cap, D), dtype=view.dtype)
    V = np.zeros_like(K)
    IK = np.zeros((S, cap, layout.idx_dim), dtype=view.dtype) if layout.idx_dim else None
    for s, L in enumerate(lens):
        for h in range(layout.n_kv_heads):
            for p in range(L):
                o = row_offset(table, layout.page_pos, pe, s, h, p, D)
                K[s, h, p] = view[o + layout.k_off // es: o + layout.k_off // es + D]
                V[s, h, p] = view[o + layout.v_off // es: o + layout.v_off // es + D]
        if IK is not None:
            DI = layout.idx_dim
            for p in range(L):
                o = row_offset(table, layout.page_pos, pe, s, 0, p, DI) + layout.ik_off // es
                IK[s, p] = view[o:o + DI]
    return K, V, IK


def read_pooled(layout: PageLayout, table, arena: np.ndarray, s: int, n_blocks: int) -> np.ndarray:
    """Read the float32 pooled rows of blocks 0..n_blocks-1 of stream s from the arena."""
    f32 = arena.view(np.float32)
    pe32 = layout.page_bytes // 4
    DI = layout.idx_dim
    out = np.zeros((n_blocks, DI), dtype=np.float32)
    for b in range(n_blocks):
        o = pool_row_offset(table, layout.page_pos, pe32, s, b, DI) + layout.pool_off // 4
        out[b] = f32[o:o + DI]
    return out


# ---------------------------------------------------------------------------
# Attention (decode, prefill, sparse)
# ---------------------------------------------------------------------------

def _softmax_rows_attend(z: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Textbook softmax attention in float64: w = exp(z - max z); out = (w V) / sum w."""
    m = np.max(z, axis=-1, keepdims=True)
    w = np.exp(z - m)
    return (w @ V) / np.sum(w, axis=-1, keepdims=True)


def decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, lens: Sequence[int], scale: float) -> np.ndarray:
    """Dense decode attention, float64.

    q [S][Hq][D], K/V [S][Hkv][cap][D] (exact input values as float64).
    Query head h reads KV head h // (Hq/Hkv) over all cached positions 0..L-1
    (the current token is already stored).  A stream with L = 0 gives a zero
    row.  (The pages fix none of these three points; these are the readings.)
    [P1 "What this changes"]: fn_attn_chunks produces the dense attention rows.
    """
    S, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        for h in range(Hq):
            g = h // G
            z = scale * (K[s, g, :L] @ q[s, h])
            out[s, h] = _softmax_rows_attend(z[None, :], V[s, g, :L])[0]
    return out


def decode_window(q: np.ndarray, K: np.ndarray, V: np.ndarray, lens: Sequence[int], scale: float) -> np.ndarray:
    """Decode of a window of W query tokens at the end of each stream's cache, float64.

    q [S][W][Hq][D], K/V [S][Hkv][cap][D].  Query w of stream s stands at
    position L - W + w and attends to keys 0 .. L - W + w; a query with no key
    (L - W + w < 0) gives a zero row.  [P1 "What this changes"] names
    fn_attn_chunks_ahead beside fn_attn_chunks and nothing more: the reading is
    the drafted-token form of decode, several new tokens verified at once, each
    seeing the cache up to itself.
    """
    S, W, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, W, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        for w in range(W):
            last = L - W + w          # the query's own position
            if last < 0:
                continue
            for h in range(Hq):
                g = h // G
                z = scale * (K[s, g, :last + 1] @ q[s, w, h])
                out[s, w, h] = _softmax_rows_attend(z[None, :], V[s, g, :last + 1])[0]
    return out


def prefill(q: np.ndarray, K: np.ndarray, V: np.ndarray, q_pos0: int, scale: float, causal: bool = True,
            rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Causal prompt attention for one chunk of queries, float64.

    q [Nq][Hq][D] are the queries at absolute positions q_pos0 .. q_pos0+Nq-1;
    K/V [Hkv][cap][D] hold positions 0 .. q_pos0+Nq-1 (stored before the chunk).
    Query at position p attends to keys j <= p (the causal reading); without the mask
    to every key 0 .. q_pos0+Nq-1.  ``rows`` limits the work to some query rows
    (the result still has Nq rows; others are zero).
    """
    Nq, Hq, D = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    Lk = q_pos0 + Nq
    out = np.zeros((Nq, Hq, D), dtype=np.float64)
    sel = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    if len(sel) == 0:
        return out
    for h in range(Hq):
        g = h // G
        Kg = K[g, :Lk]
        Vg = V[g, :Lk]
        z = scale * (q[sel, h] @ Kg.T)            # [n][Lk]
        if causal:
            pos = q_pos0 + sel
            mask = np.arange(Lk)[None, :] > pos[:, None]
            z = np.where(mask, -np.inf, z)
        out[sel, h] = _softmax_rows_attend(z, Vg)
    return out


def sparse(q: np.ndarray, K: np.ndarray, V: np.ndarray, block_ids: Sequence[Sequence[int]], scale: float) -> np.ndarray:
    """Attention over the selected blocks only, float64.

    Block b covers positions 4b .. 4b+3 ([P1 "What this changes"]: pooled rows
    of blocks of four).  The rows attended are those positions of the selected
    blocks, in ascending position order; with no selected block the row is zero.
    """
    S, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        ids = sorted(int(b) for b in block_ids[s])
        if not ids:
            continue
        pos = np.array([4 * b + j for b in ids for j in range(4)], dtype=np.int64)
        for h in range(Hq):
            g = h // G
            z = scale * (K[s, g, pos] @ q[s, h])
            out[s, h] = _softmax_rows_attend(z[None, :], V[s, g, pos])[0]
    return out


# ---------------------------------------------------------------------------
# Block pooling, block scores, top-k
# ---------------------------------------------------------------------------

def pool(IK: np.ndarray, lens: Sequence[int]) -> list:
    """Mean of the indexer-key rows of each complete block of four positions.

    IK [S][cap][DI] exact values as float64.  For b < floor(L/4):
    pooled[b] = float32(((IK[4b] + IK[4b+1]) + IK[4b+2]) + IK[4b+3]) / 4)
    with the sum in float64 (exact for bf16 rows whose exponents lie within 43
    binades), one rounding to float32.  Readings: the pooled rows are means of
    the 128-wide indexer-key rows; the sum is exact and rounded once; only
    complete blocks are pooled.
    [P1 "What this changes"]: the pool kernel reads once per block of four and
    the page holds the pooled rows of its n/4 blocks.
    Returns a list of [nb_s][DI] float32 arrays.
    """
    out = []
    for s, L in enumerate(lens):
        nb = int(L) // 4
        x = IK[s, :4 * nb].reshape(nb, 4, IK.shape[-1])
        acc = ((x[:, 0] + x[:, 1]) + x[:, 2]) + x[:, 3]
        out.append((acc * 0.25).astype(np.float32))
    return out


def scores(qI: np.ndarray, pooled: np.ndarray) -> np.ndarray:
    """Block scores: sum over indexer heads of the dot product of the head's
    indexer query with the block's pooled row, in float64.

    qI [Hi][DI] exact values (float64), pooled [nb][DI] float32.
    Order (the pages fix none; this is the reading).  In exact arithmetic
    sum_h sum_d qI[h,d] p[d] = sum_d (sum_h qI[h,d]) p[d], so the queries are
    first summed over the heads, head by head, into q[d]; every product
    p[d] * q[d] is rounded to float64; the products are added in 8 groups, group
    j holding the dims of the 4-dim chunks c = j, j+8, j+16, ... (dims 4c .. 4c+3)
    in increasing dim order from 0; and the 8 group sums meet in the fixed tree
    ((g0 + g1) + (g2 + g3)) + ((g4 + g5) + (g6 + g7)).  Only the rounding order is
    chosen; the value is the definition's to float64 precision.
    """
    P = pooled.astype(np.float64)
    nb = P.shape[0]
    Hi, DI = qI.shape
    q = np.zeros(DI, dtype=np.float64)
    for h in range(Hi):
        q = q + qI[h]
    prod = P * q[None, :]
    groups = []
    for j in range(8):
        acc = np.zeros(nb, dtype=np.float64)
        for c in range(j, (DI + 3) // 4, 8):
            for d in range(4 * c, min(4 * c + 4, DI)):
                acc = acc + prod[:, d]
        groups.append(acc)
    g = groups
    return ((g[0] + g[1]) + (g[2] + g[3])) + ((g[4] + g[5]) + (g[6] + g[7]))


def topk(score: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k highest scores, lowest id first among equal scores, returned ascending.

    Orders by (score descending, id ascending); -0.0 equals +0.0; when there are
    no more than k blocks every block is selected.  (The pages fix only
    "lowest index wins ties"; the rest are readings.)
    """
    nb = score.shape[0]
    ids = np.arange(nb)
    order = np.lexsort((ids, -score))
    return np.sort(order[:min(k, nb)])


# ---------------------------------------------------------------------------
# e4m3 rows with one float32 scale a row
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(codes) -> np.ndarray:
    """Value of each e4m3 code as float64, from the format's definition.

    OCP 8-bit floating point, E4M3 ("fn": finite only): bit 7 is the sign,
    bits 6..3 the exponent with bias 7, bits 2..0 the mantissa.  An exponent
    field of 0 is subnormal, m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7).
    S.1111.111 is NaN; there are no infinities, so S.1111.110 = 448 is the
    largest magnitude.  [P2 commit 5c09685]: rows hold e4m3 codes, and
    the check computes each value as code times scale in float64.
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(y) -> np.ndarray:
    """e4m3 code of each float32 value: the nearest finite e4m3 value, ties to
    the even code; magnitudes beyond 448 become 448; the sign bit is kept (so
    -0.0 -> 0x80).  NaN is not accepted.

    Readings: round to nearest even, as for every IEEE-style narrowing; the
    pages' store saturates rather than producing NaN (the format has no
    infinity).  Done by brute force over the table of the 127 non-negative
    finite values (codes 0..126, which increase with the code).
    """
    y = np.asarray(y, dtype=np.float32)
    assert not np.isnan(y).any()
    table = e4m3_value(np.arange(127))
    mag = np.minimum(np.abs(y.astype(np.float64)), E4M3_MAX).reshape(-1)
    out = np.empty(mag.shape, dtype=np.int64)
    step = 1 << 14
    for i in range(0, mag.size, step):
        d = np.abs(mag[i:i + step, None] - table[None, :])     # exact in float64
        best = np.argmin(d, axis=1)                              # the lower code on a tie
        nxt = np.minimum(best + 1, 126)
        tie = (d[np.arange(best.size), nxt] == d[np.arange(best.size), best]) & (nxt != best)
        best = np.where(tie & (best % 2 == 1), nxt, best)       # the even one of the two
        out[i:i + step] = best
    sign = np.signbit(y.reshape(-1)).astype(np.int64) << 7
    return (out | sign).astype(np.uint8).reshape(y.shape)


def e4m3_quantize_rows(x) -> tuple:
    """Codes and scale of each row (last axis) of float32 values.

    scale = amax / 448 with amax = max |x| over the row, a float32 quotient;
    code = e4m3_encode(x / scale), float32 quotients; a row of zeros gets scale
    0 and codes 0.  [P2 commit 5c09685] names the store (codes plus an fp32
    scale a row) but not the scale rule: this absmax-to-448 rule is the
    reading, so that code x scale spans the row's range.  Returns (codes
    uint8 [..., D], scales float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    live = amax > 0
    div = np.where(live, scale, np.float32(1.0)).astype(np.float32)
    codes = e4m3_encode((x / div[..., None]).astype(np.float32))
    codes = np.where(live[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, np.where(live, scale, np.float32(0.0)).astype(np.float32)


def e4m3_dequantize(codes, scales) -> np.ndarray:
    """code x scale in float64 (exact: 4 significant bits times 24)."""
    return e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def place_fp8(layout: PageLayout, table, n_pages: int, lens: Sequence[int], KC, VC, KS, VS) -> np.ndarray:
    """Write e4m3 rows and their scales into a fresh zero arena (bytes) through the table.

    KC, VC: [S][Hkv][cap][D] uint8 codes; KS, VS: [S][Hkv][cap] float32 scales.
    A row's codes sit at row_offset(..., width=D) in the code regions and its
    scale at row_offset(..., width=4) (bytes) in the scale regions: the same
    page lookup, rows of 4 bytes.
    """
    assert layout.dtype == "fp8"
    arena = np.zeros(n_pages * layout.page_bytes, dtype=np.uint8)
    D = layout.head_dim
    pe = layout.page_elems
    for s, L in enumerate(lens):
        for h in range(layout.n_kv_heads):
            for p in range(int(L)):
                o = row_offset(table, layout.page_pos, pe, s, h, p, D)
                arena[layout.k_off + o:layout.k_off + o + D] = KC[s, h, p]
                arena[layout.v_off + o:layout.v_off + o + D] = VC[s, h, p]
                so = row_offset(table, layout.page_pos, pe, s, h, p, 4)
                arena[layout.ks_off + so:layout.ks_off + so + 4] = np.frombuffer(np.float32(KS[s, h, p]).tobytes(), np.uint8)
                arena[layout.vs_off + so:layout.vs_off + so + 4] = np.frombuffer(np.float32(VS[s, h, p]).tobytes(), np.uint8)
    return arena


def gather_fp8(layout: PageLayout, table, arena: np.ndarray, lens: Sequence[int], cap: Optional[int] = None):
    """Inverse of place_fp8(): (KC, VC, KS, VS) read one row at a time through row_offset()."""
    D = layout.head_dim
    pe = layout.page_elems
    cap = int(cap if cap is not None else max(list(lens) + [1]))
    S, H = len(lens), layout.n_kv_heads
    KC = np.zeros((S, H, cap, D), dtype=np.uint8)
    VC = np.zeros_like(KC)
    KS = np.zeros((S, H, cap), dtype=np.float32)
    VS = np.zeros_like(KS)
    for s, L in enumerate(lens):
        for h in range(H):
            for p in range(int(L)):
                o = row_offset(table, layout.page_pos, pe, s, h, p, D)
                KC[s, h, p] = arena[layout.k_off + o:layout.k_off + o + D]
                VC[s, h, p] = arena[layout.v_off + o:layout.v_off + o + D]
                so = row_offset(table, layout.page_pos, pe, s, h, p, 4)
                KS[s, h, p] = arena[layout.ks_off + so:layout.ks_off + so + 4].view(np.float32)[0]
                VS[s, h, p] = arena[layout.vs_off + so:layout.vs_off + so + 4].view(np.float32)[0]
    return KC, VC, KS, VS
