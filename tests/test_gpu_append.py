"""GPU parity of paged_kv_append: a step's K, V and indexer-key rows stored through the table and
the pooled rows of the blocks the step completes, against the oracle's placement and pooling.

TensorFold PR #1169 "Receipt": stored rows and pooled rows match the contiguous layout, and the
guards are left untouched.
Bar: the arena after a sequence of appends equals, byte for byte, the oracle's arena (rows placed
through its own row addressing, pooled rows from its own float64 pooling).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import paged_kv_cache_pg_amd as P  # noqa: E402
from paged_kv_cache_pg_amd.inputs import make_workload  # noqa: E402
from gpu_util import dev, host_bytes  # noqa: E402

HKV, D, DI = 4, 256, 128
GUARD = 4096


def _expected_arena(w, table, n_pages, page_pos, with_ik=True):
    olay = O.PageLayout(HKV, D, page_pos, w.dtype, idx_dim=DI)
    arena = O.place(olay, table, n_pages, w.lens, w.K, w.V, w.IK if with_ik else None)
    if with_ik:
        f32 = arena.view(np.float32)
        pooled = O.pool(w.as_f64("IK"), w.lens)
        pe32 = olay.page_bytes // 4
        for s, L in enumerate(w.lens):
            for b in range(L // 4):
                o = O.pool_row_offset(table, page_pos, pe32, s, b, DI) + olay.pool_off // 4
                f32[o:o + DI] = pooled[s][b]
    return arena


def _append_all(w, table, n_pages, page_pos, steps, with_ik=True, max_len=None):
    """Apply appends of the given sizes (every stream appends the same count; a finished stream is
    given pos0 = max_len so its rows are dropped)."""
    S = w.n_streams
    lay = P.ArenaLayout(HKV, D, page_pos, P.PAGED_BF16, idx_dim=DI)
    buf = torch.full((n_pages * lay.page_bytes + 2 * GUARD,), 0, dtype=torch.uint8, device="cuda")
    buf[:GUARD] = 0xA5
    buf[-GUARD:] = 0xA5
    base = buf.data_ptr() + GUARD
    tt = dev(table.astype(np.int32)) if table is not None else None
    pg = P.make_pg(tt, page_pos, lay.page_elems)
    kv = P.make_kv(base + lay.k_off, base + lay.v_off, P.PAGED_BF16, HKV, D)
    max_len = max_len if max_len is not None else max(w.lens)
    pos = [0] * S
    for n in steps:
        kn = np.zeros((S, n, HKV, D), np.uint16)
        vn = np.zeros_like(kn)
        ikn = np.zeros((S, n, DI), np.uint16)
        p0 = []
        for s, L in enumerate(w.lens):
            m = max(0, min(n, L - pos[s]))
            assert m in (0, n), "a step must not run past a stream's length"
            if m:
                kn[s, :m] = w.K[s, :, pos[s]:pos[s] + m].transpose(1, 0, 2)
                vn[s, :m] = w.V[s, :, pos[s]:pos[s] + m].transpose(1, 0, 2)
                ikn[s, :m] = w.IK[s, pos[s]:pos[s] + m]
            p0.append(pos[s] if pos[s] < L else max_len)
        P.paged_kv_append(dev(kn), dev(vn), dev(ikn) if with_ik else None, n, kv, base + lay.ik_off,
                          base + lay.pool_off, DI, pg, dev(np.array(p0, np.int32)), S, max_len)
        pos = [min(L, p + n) for p, L in zip(pos, w.lens)]
    torch.cuda.synchronize()
    b = host_bytes(buf)
    assert np.all(b[:GUARD] == 0xA5) and np.all(b[-GUARD:] == 0xA5), "guards overwritten"
    return b[GUARD:len(b) - GUARD]


@pytest.mark.parametrize("ptok", [16, 48, 256])
def test_append_steps_equal_oracle_arena(ptok):
    L = 1000
    w = make_workload(71, [L, L], ptok, 16, HKV, dtype="bf16", table_kind="shuffled", idx_dim=DI, n_idx_heads=4)
    steps = [7, 1, 1, 2, 64, 300, 3, 1, 621]          # sums to 1000: blocks complete inside and across steps
    assert sum(steps) == L
    got = _append_all(w, w.table, w.n_pages, ptok, steps)
    want = _expected_arena(w, w.table, w.n_pages, ptok)
    assert np.array_equal(got, want)


def test_append_contiguous_and_one_token_steps():
    """No table (contiguous form; rows a head a multiple of 4), one token a step for 64 steps (a decode loop)."""
    L = 64
    w = make_workload(72, [L, L, L], 16, 16, HKV, dtype="bf16", table_kind=None, idx_dim=DI, n_idx_heads=4)
    got = _append_all(w, None, 3, L, [1] * L)
    want = _expected_arena(w, None, 3, L)
    assert np.array_equal(got, want)


def test_append_without_indexer_keys_writes_only_k_and_v():
    L = 200
    w = make_workload(73, [L, L], 48, 16, HKV, dtype="bf16", table_kind="shuffled", idx_dim=DI, n_idx_heads=4)
    got = _append_all(w, w.table, w.n_pages, 48, [50, 150], with_ik=False)
    want = _expected_arena(w, w.table, w.n_pages, 48, with_ik=False)
    assert np.array_equal(got, want)


def test_append_one_prefill_chunk_of_2048():
    """A prefill chunk: 2048 tokens into pages of 256 in one launch, after 100 earlier tokens."""
    L = 2148
    w = make_workload(74, [L], 256, 32, HKV, dtype="bf16", table_kind="shuffled", idx_dim=DI, n_idx_heads=4)
    got = _append_all(w, w.table, w.n_pages, 256, [100, 2048])
    want = _expected_arena(w, w.table, w.n_pages, 256)
    assert np.array_equal(got, want)
