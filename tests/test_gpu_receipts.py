"""The pages' receipt gates applied to every call of the path, not only dense decode.

TensorFold PR #1169 "Receipt": guards and inputs stay intact, stores and pooled rows
equal contiguous, a batch gives each stream what it gives alone ("concurrent == solo"),
and a kept state restored into pages resumes to the same bytes as a fresh one.  PR #2244
"What this changes": grouped lanes built without their own page table read and wrote
other streams' pages, the class of bug a batch-versus-solo comparison catches.  PR #1170
("What this changes", "Receipt"): kept states move between the paged and the contiguous
forms and are restored into a lane's pages.

Every comparison here is bit for bit: the same kernel over the same rows must give the
same bytes whatever else shares the launch, whatever table the rows were restored under.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import paged_kv_cache_pg_amd as P  # noqa: E402
from paged_kv_cache_pg_amd.inputs import (  # noqa: E402
    draw_e4m3_codes, draw_row_scales, f32_to_bf16_bits, make_table, make_workload)
from gpu_util import (Placed, PlacedFp8, dev, guarded_out, host_bytes, out_guards_intact, rel_err_rows,  # noqa: E402
                      TOL)

HQ, HKV, DI, HI, D = 32, 4, 128, 4, 256


def _qsa(seed, lens, ptok, table_kind="shuffled"):
    return make_workload(seed, lens, ptok, HQ, HKV, dtype="bf16", table_kind=table_kind, idx_dim=DI, n_idx_heads=HI)


def _guarded(n, dtype, guard=256):
    """A device buffer of n elements between two canary bands: (whole buffer, the n-element view)."""
    buf = torch.empty(n + 2 * guard, dtype=dtype, device="cuda")
    buf.view(torch.uint8).fill_(0x5A)
    return buf, buf[guard:guard + n]


def _canaries_intact(buf, guard=256):
    b = host_bytes(buf)
    es = buf.element_size()
    return bool(np.all(b[:guard * es] == 0x5A) and np.all(b[len(b) - guard * es:] == 0x5A))


def _pool_all(pl, lens, max_len=None):
    S = len(lens)
    b0 = dev(np.zeros(S, np.int32))
    b1 = dev(np.array([L // 4 for L in lens], np.int32))
    P.paged_pool_blocks(pl.ik, pl.pooled, DI, P.PAGED_BF16, pl.pg, b0, b1, S, max_len or max(lens))


def _topk_call(pl, qi, lens_d, S, max_len, k, ids, cnt, sc):
    ws = torch.empty(P.paged_topk_workspace(S, max_len, k), dtype=torch.uint8, device="cuda")
    P.paged_block_scores_topk(qi, P.PAGED_BF16, HI, DI, pl.pooled, P.PAGED_BF16, pl.pg, lens_d, S, max_len, k, ids,
                              cnt, sc, ws)


def _sparse_call(q, kv, pg, ids, cnt, k, S, max_len, out):
    ws = torch.zeros(P.paged_sparse_attn_workspace(S, HQ, k), dtype=torch.uint8, device="cuda")
    P.paged_sparse_attn(q, P.PAGED_BF16, HQ, kv, pg, ids, cnt, k, S, max_len, 1 / 16, out, ws)


# ---------------------------------------------------------------------------
# guards and inputs intact
# ---------------------------------------------------------------------------

def test_pool_changes_only_the_pooled_rows_it_owns():
    """Pooling blocks [b0, b1) of each stream writes exactly those blocks' pooled rows (equal to the
    oracle's) and no other byte of the arena or of the guard bands around it."""
    lens = [3000, 1700, 999]
    w = _qsa(71, lens, 48)
    pl = Placed(w)
    before = pl.arena_now().copy()
    begin, end = [5, 0, 100], [700, 425, 249]
    b0, b1 = dev(np.array(begin, np.int32)), dev(np.array(end, np.int32))
    P.paged_pool_blocks(pl.ik, pl.pooled, DI, P.PAGED_BF16, pl.pg, b0, b1, 3, max(lens))
    torch.cuda.synchronize()
    assert pl.guards_intact()
    want = before.copy()
    f32 = want.view(np.float32)
    pooled = O.pool(w.as_f64("IK"), lens)
    pe32 = pl.olay.page_bytes // 4
    for s in range(3):
        for b in range(begin[s], end[s]):
            o = O.pool_row_offset(w.table, 48, pe32, s, b, DI) + pl.olay.pool_off // 4
            f32[o:o + DI] = pooled[s][b]
    assert np.array_equal(pl.arena_now(), want)


def test_scores_topk_leave_the_arena_and_the_outputs_neighbours_alone():
    """Scores + top-k read the arena and write only ids, counts and scores: the arena is unchanged
    byte for byte, the canaries around each output survive, and the outputs equal the oracle's."""
    lens = [8192, 5000, 1000]
    w = _qsa(72, lens, 256)
    pl = Placed(w)
    _pool_all(pl, lens)
    torch.cuda.synchronize()
    before = pl.arena_now().copy()
    S, ml, k = 3, max(lens), 300
    ibuf, ids = _guarded(S * k, torch.int32)
    cbuf, cnt = _guarded(S, torch.int32)
    sbuf, sc = _guarded(S * (ml // 4), torch.float64)
    _topk_call(pl, dev(w.qI), pl.lens, S, ml, k, ids, cnt, sc)
    torch.cuda.synchronize()
    assert pl.guards_intact() and np.array_equal(pl.arena_now(), before)
    for b in (ibuf, cbuf, sbuf):
        assert _canaries_intact(b)
    ids, cnt, sc = ids.cpu().numpy().reshape(S, k), cnt.cpu().numpy(), sc.cpu().numpy().reshape(S, ml // 4)
    pooled = O.pool(w.as_f64("IK"), lens)
    for s, L in enumerate(lens):
        want_sc = O.scores(w.as_f64("qI")[s], pooled[s])
        assert np.array_equal(sc[s, :L // 4].view(np.uint64), want_sc.view(np.uint64))
        want = O.topk(want_sc, k)
        n = len(want)                       # a stream of fewer than k blocks selects them all
        assert cnt[s] == n and np.array_equal(ids[s, :n], want) and np.all(ids[s, n:] == -1)


def test_sparse_attention_leaves_arena_ids_and_neighbours_alone():
    lens = [4096, 2000]
    w = _qsa(73, lens, 48)
    pl = Placed(w)
    before = pl.arena_now().copy()
    k = 96
    rng = np.random.default_rng(73)
    ids_np = np.stack([np.sort(rng.choice(L // 4, k, replace=False)) for L in lens]).astype(np.int32)
    cnt_np = np.array([k, 80], np.int32)
    ids_d, cnt_d = dev(ids_np), dev(cnt_np)
    obuf, out = guarded_out((2, HQ, D))
    _sparse_call(dev(w.q), pl.kv, pl.pg, ids_d, cnt_d, k, 2, max(lens), out)
    torch.cuda.synchronize()
    assert out_guards_intact(obuf)
    assert pl.guards_intact() and np.array_equal(pl.arena_now(), before)
    assert np.array_equal(ids_d.cpu().numpy(), ids_np) and np.array_equal(cnt_d.cpu().numpy(), cnt_np)
    sel = [list(ids_np[s, :cnt_np[s]]) for s in range(2)]
    ref = O.sparse(w.as_f64("q"), w.as_f64("K"), w.as_f64("V"), sel, 1 / 16)
    assert rel_err_rows(out.cpu().numpy(), ref) <= TOL


def test_rows_gather_writes_only_the_rows_asked_for():
    """A gather of positions [begin, end) into a strided contiguous buffer: the arena is unchanged,
    the gathered rows equal the workload's, and every other row of the buffer (positions outside the
    range, padding heads) and the canaries around it keep their bytes."""
    lens = [3000, 1234]
    w = make_workload(74, lens, 48, 16, 4, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    before = pl.arena_now().copy()
    S, H, cap = 2, 4, 3100
    Hpad = 5                                    # a padding head between the heads' blocks is never written
    n = S * Hpad * cap * D
    buf, dst = _guarded(n, torch.int16)
    begin, end = [100, 0], [2900, 1234]
    P.paged_rows_gather(dst, Hpad * cap * D, cap * D, D, pl.base + pl.lay.k_off, H, D, P.PAGED_BF16, pl.pg,
                        dev(np.array(begin, np.int32)), dev(np.array(end, np.int32)), S, max(lens))
    torch.cuda.synchronize()
    assert _canaries_intact(buf)
    assert pl.guards_intact() and np.array_equal(pl.arena_now(), before)
    got = dst.cpu().numpy().view(np.uint16).reshape(S, Hpad, cap, D)
    untouched = np.full((D,), 0x5A5A, np.uint16)
    for s in range(S):
        assert np.array_equal(got[s, :H, begin[s]:end[s]], w.K[s, :, begin[s]:end[s]])
        assert np.all(got[s, :H, :begin[s]] == untouched) and np.all(got[s, :H, end[s]:] == untouched)
        assert np.all(got[s, H:] == untouched)


# ---------------------------------------------------------------------------
# concurrent == solo
# ---------------------------------------------------------------------------

def _solo_pg(pl, s, page_pos, page_elems):
    table1 = pl.table[s:s + 1].contiguous()
    return table1, P.make_pg(table1, page_pos, page_elems)


def test_sparse_attention_concurrent_equals_solo():
    lens = [8192, 3000, 700]
    w = _qsa(75, lens, 48)
    pl = Placed(w)
    k = 160
    rng = np.random.default_rng(75)
    ids_np = np.full((3, k), -1, np.int32)
    cnt_np = np.array([k, 120, k], np.int32)
    for s, L in enumerate(lens):
        ids_np[s, :cnt_np[s]] = np.sort(rng.choice(L // 4, cnt_np[s], replace=False))
    q = dev(w.q)
    out = torch.empty((3, HQ, D), dtype=torch.float32, device="cuda")
    _sparse_call(q, pl.kv, pl.pg, dev(ids_np), dev(cnt_np), k, 3, max(lens), out)
    torch.cuda.synchronize()
    batch = out.cpu().numpy()
    for s in range(3):
        table1, pg1 = _solo_pg(pl, s, 48, pl.lay.page_elems)
        o1 = torch.empty((1, HQ, D), dtype=torch.float32, device="cuda")
        _sparse_call(q[s:s + 1].contiguous(), pl.kv, pg1, dev(ids_np[s:s + 1]), dev(cnt_np[s:s + 1]), k, 1, lens[s],
                     o1)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy()[0].view(np.uint32), batch[s].view(np.uint32)), s


def test_scores_topk_concurrent_equals_solo():
    lens = [16384, 6000, 800]
    w = _qsa(76, lens, 256)
    pl = Placed(w)
    _pool_all(pl, lens)
    S, ml, k = 3, max(lens), 200
    qi = dev(w.qI)
    ids = torch.empty((S, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(S, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, ml // 4), dtype=torch.float64, device="cuda")
    _topk_call(pl, qi, pl.lens, S, ml, k, ids, cnt, sc)
    torch.cuda.synchronize()
    ids, cnt, sc = ids.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()
    for s, L in enumerate(lens):
        table1, pg1 = _solo_pg(pl, s, 256, pl.lay.page_elems)
        i1 = torch.empty((1, k), dtype=torch.int32, device="cuda")
        c1 = torch.empty(1, dtype=torch.int32, device="cuda")
        s1 = torch.zeros((1, L // 4), dtype=torch.float64, device="cuda")
        ws = torch.empty(P.paged_topk_workspace(1, L, k), dtype=torch.uint8, device="cuda")
        P.paged_block_scores_topk(qi[s:s + 1].contiguous(), P.PAGED_BF16, HI, DI, pl.pooled, P.PAGED_BF16, pg1,
                                  pl.lens[s:s + 1].contiguous(), 1, L, k, i1, c1, s1, ws)
        torch.cuda.synchronize()
        assert np.array_equal(i1.cpu().numpy()[0], ids[s]) and c1.item() == cnt[s], s
        assert np.array_equal(s1.cpu().numpy()[0].view(np.uint64), sc[s, :L // 4].view(np.uint64)), s


def test_window_concurrent_equals_solo():
    lens, W, hq, hkv = [9000, 130, 3], 2, 16, 4
    w = make_workload(77, lens, 48, hq, hkv, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    rng = np.random.default_rng(77)
    q = dev(f32_to_bf16_bits(rng.standard_normal((3, W, hq, D), dtype=np.float32)))

    def window(qq, pg, lens_d, S, max_len):
        ws = torch.zeros(max(16, P.paged_attn_decode_window_workspace(S, hq, W, max_len)), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((S, W, hq, D), dtype=torch.float32, device="cuda")
        P.paged_attn_decode_window(qq, P.PAGED_BF16, hq, W, pl.kv, pg, lens_d, S, max_len, 1 / 16, out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    batch = window(q, pl.pg, pl.lens, 3, max(lens))
    for s in range(3):
        table1, pg1 = _solo_pg(pl, s, 48, pl.lay.page_elems)
        o1 = window(q[s:s + 1].contiguous(), pg1, pl.lens[s:s + 1].contiguous(), 1, lens[s])
        assert np.array_equal(o1[0].view(np.uint32), batch[s].view(np.uint32)), s


def test_fp8_decode_concurrent_equals_solo():
    lens, hq, hkv, ptok = [5000, 700, 64], 32, 4, 64
    rng = np.random.default_rng(78)
    S = len(lens)
    cap = max(lens)
    q = f32_to_bf16_bits(rng.standard_normal((S, hq, D), dtype=np.float32))
    KC = draw_e4m3_codes(rng, (S, hkv, cap, D))
    VC = draw_e4m3_codes(rng, (S, hkv, cap, D))
    KS = draw_row_scales(rng, (S, hkv, cap))
    VS = draw_row_scales(rng, (S, hkv, cap))
    table, n_pages = make_table("shuffled", [(L + ptok - 1) // ptok for L in lens], rng)
    pl = PlacedFp8(lens, hkv, ptok, KC, VC, KS, VS, table=table, n_pages=n_pages)
    qd = dev(q)

    def run(qq, pg, lens_d, n, max_len):
        ws = torch.zeros(P.paged_attn_decode_workspace(n, hq, max_len), dtype=torch.uint8, device="cuda")
        out = torch.empty((n, hq, D), dtype=torch.float32, device="cuda")
        P.paged_attn_decode(qq, P.PAGED_BF16, hq, pl.kv, pg, lens_d, n, max_len, 1 / 16, out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    batch = run(qd, pl.pg, pl.lens, S, cap)
    for s in range(S):
        table1, pg1 = _solo_pg(pl, s, ptok, pl.lay.page_elems)
        o1 = run(qd[s:s + 1].contiguous(), pg1, pl.lens[s:s + 1].contiguous(), 1, lens[s])
        assert np.array_equal(o1[0].view(np.uint32), batch[s].view(np.uint32)), s


# ---------------------------------------------------------------------------
# resumed == fresh
# ---------------------------------------------------------------------------

def test_page_runs_restored_under_another_table_resume_bit_for_bit():
    """Save every K, V and indexer-key row of a batch (gathered through table T1 into the contiguous
    layout), restore them into a zeroed arena through a different shuffled table T2, and resume:
    dense decode, pooling, scores + top-k and sparse attention over the restored pages give the
    same bytes as over the original ones."""
    lens = [4096, 2500, 517]
    ptok = 48
    w = _qsa(79, lens, ptok)
    pl = Placed(w)
    S, L = len(lens), max(lens)
    lay = pl.lay
    zero = dev(np.zeros(S, np.int32))
    cont = {name: torch.zeros(shape, dtype=torch.int16, device="cuda")
            for name, shape in (("K", (S, HKV, L, D)), ("V", (S, HKV, L, D)), ("IK", (S, L, DI)))}
    regions = (("K", lay.k_off, HKV, D, HKV * L * D, L * D), ("V", lay.v_off, HKV, D, HKV * L * D, L * D),
               ("IK", lay.ik_off, 1, DI, L * DI, 0))
    for name, off, heads, width, ss, sh in regions:
        P.paged_rows_gather(cont[name], ss, sh, width, pl.base + off, heads, width, P.PAGED_BF16, pl.pg, zero,
                            pl.lens, S, L)
    # T2: another permutation of the same number of pages, in a fresh zeroed arena
    rng = np.random.default_rng(179)
    perm = rng.permutation(w.n_pages)
    t2 = np.full_like(w.table, 0)
    for s in range(S):
        for i in range(w.table.shape[1]):
            t2[s, i] = perm[w.table[s, i]]
    assert not np.array_equal(t2, w.table)
    arena2 = torch.zeros(w.n_pages * lay.page_bytes, dtype=torch.uint8, device="cuda")
    t2_d = dev(t2.astype(np.int32))
    pg2 = P.make_pg(t2_d, ptok, lay.page_elems)
    b2 = arena2.data_ptr()
    for name, off, heads, width, ss, sh in regions:
        P.paged_rows_store(cont[name], ss, sh, width, b2 + off, heads, width, P.PAGED_BF16, pg2, zero, pl.lens, S, L)
    kv2 = P.make_kv(b2 + lay.k_off, b2 + lay.v_off, P.PAGED_BF16, HKV, D)
    torch.cuda.synchronize()
    q, qi = dev(w.q), dev(w.qI)

    def resume(kv, pg, base):
        ws = torch.zeros(P.paged_attn_decode_workspace(S, HQ, L), dtype=torch.uint8, device="cuda")
        dense = torch.empty((S, HQ, D), dtype=torch.float32, device="cuda")
        P.paged_attn_decode(q, P.PAGED_BF16, HQ, kv, pg, pl.lens, S, L, 1 / 16, dense, ws)
        b1 = dev(np.array([x // 4 for x in lens], np.int32))
        P.paged_pool_blocks(base + lay.ik_off, base + lay.pool_off, DI, P.PAGED_BF16, pg, zero, b1, S, L)
        k = 100
        ids = torch.empty((S, k), dtype=torch.int32, device="cuda")
        cnt = torch.empty(S, dtype=torch.int32, device="cuda")
        sc = torch.zeros((S, L // 4), dtype=torch.float64, device="cuda")
        tws = torch.empty(P.paged_topk_workspace(S, L, k), dtype=torch.uint8, device="cuda")
        P.paged_block_scores_topk(qi, P.PAGED_BF16, HI, DI, base + lay.pool_off, P.PAGED_BF16, pg, pl.lens, S, L, k,
                                  ids, cnt, sc, tws)
        sp = torch.empty((S, HQ, D), dtype=torch.float32, device="cuda")
        _sparse_call(q, kv, pg, ids, cnt, k, S, L, sp)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in (dense, ids, cnt, sc, sp)]

    fresh = resume(pl.kv, pl.pg, pl.base)
    resumed = resume(kv2, pg2, b2)
    for a, b in zip(fresh, resumed):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # the restored arena holds each row at the place T2 gives it: the oracle's placement under T2
    want = O.place(pl.olay, t2, w.n_pages, lens, w.K, w.V, w.IK)
    got = arena2.cpu().numpy()
    pool_lo = pl.olay.pool_off
    for p in range(w.n_pages):      # rows compare everywhere but the pooled region (written by the pool call)
        a0 = p * lay.page_bytes
        assert np.array_equal(got[a0:a0 + pool_lo], want[a0:a0 + pool_lo]), p


def test_fp8_rows_restored_under_another_table_resume_bit_for_bit():
    """e4m3 codes and their row scales saved through T1 and restored through another table T2 (codes
    as byte rows, scales as 4-byte rows): decode over the restored pages gives the same bytes."""
    lens, hq, hkv, ptok = [3000, 1100], 32, 4, 64
    rng = np.random.default_rng(80)
    S, cap = len(lens), max(lens)
    q = dev(f32_to_bf16_bits(rng.standard_normal((S, hq, D), dtype=np.float32)))
    KC = draw_e4m3_codes(rng, (S, hkv, cap, D))
    VC = draw_e4m3_codes(rng, (S, hkv, cap, D))
    KS = draw_row_scales(rng, (S, hkv, cap))
    VS = draw_row_scales(rng, (S, hkv, cap))
    table, n_pages = make_table("shuffled", [(L + ptok - 1) // ptok for L in lens], rng)
    pl = PlacedFp8(lens, hkv, ptok, KC, VC, KS, VS, table=table, n_pages=n_pages)
    lay = pl.lay
    zero = dev(np.zeros(S, np.int32))
    # a code row of 256 bytes is copied as 128 bf16 slots (bit patterns, untouched)
    page_elems16 = lay.page_bytes // 2
    pg16_1 = P.make_pg(pl.table, ptok, page_elems16)
    codes = {n: torch.zeros((S, hkv, cap, D // 2), dtype=torch.int16, device="cuda") for n in ("K", "V")}
    perm = rng.permutation(n_pages)
    t2 = perm[table].astype(np.int32)
    assert not np.array_equal(t2, table)
    t2_d = dev(t2)
    pg16_2 = P.make_pg(t2_d, ptok, page_elems16)
    arena2 = torch.zeros(n_pages * lay.page_bytes, dtype=torch.uint8, device="cuda")
    b2 = arena2.data_ptr()
    # codes move through the library's row copies (a code row is 256 bytes); a scale row is 4 bytes,
    # under the 16-byte rows the copy kernel moves, so the scale regions are moved page by page on the host
    for n, off in (("K", lay.k_off), ("V", lay.v_off)):
        P.paged_rows_gather(codes[n], hkv * cap * D // 2, cap * D // 2, D // 2, pl.base + off, hkv, D // 2,
                            P.PAGED_BF16, pg16_1, zero, pl.lens, S, cap)
        P.paged_rows_store(codes[n], hkv * cap * D // 2, cap * D // 2, D // 2, b2 + off, hkv, D // 2, P.PAGED_BF16,
                           pg16_2, zero, pl.lens, S, cap)
    torch.cuda.synchronize()
    src = pl.arena_now()
    dst = arena2.cpu().numpy()
    for s, L in enumerate(lens):
        for lp in range((L + ptok - 1) // ptok):
            for off in (lay.ks_off, lay.vs_off):
                a = int(table[s, lp]) * lay.page_bytes + off
                b = int(t2[s, lp]) * lay.page_bytes + off
                dst[b:b + hkv * ptok * 4] = src[a:a + hkv * ptok * 4]
    arena2 = dev(dst)
    b2 = arena2.data_ptr()
    kv2 = P.make_kv(b2 + lay.k_off, b2 + lay.v_off, P.PAGED_FP8_E4M3, hkv, D, b2 + lay.ks_off, b2 + lay.vs_off)
    pg2 = P.make_pg(t2_d, ptok, lay.page_elems)

    def run(kv, pg):
        ws = torch.zeros(P.paged_attn_decode_workspace(S, hq, cap), dtype=torch.uint8, device="cuda")
        out = torch.empty((S, hq, D), dtype=torch.float32, device="cuda")
        P.paged_attn_decode(q, P.PAGED_BF16, hq, kv, pg, pl.lens, S, cap, 1 / 16, out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    assert np.array_equal(run(pl.kv, pl.pg).view(np.uint32), run(kv2, pg2).view(np.uint32))


# ---------------------------------------------------------------------------
# paged == contiguous on the full block-sparse workload
# ---------------------------------------------------------------------------

def test_qsa_full_size_paged_equals_contiguous():
    """3 streams x 131072 positions, pages of 256 shuffled: pooled rows, scores, top-512 ids and sparse
    attention rows from the paged arena equal those from the contiguous one, bit for bit."""
    lens = [131072] * 3
    w = _qsa(5, lens, 256)
    S, L, k = 3, 131072, 512
    results = []
    for paged in (True, False):
        pl = Placed(w, paged=paged)
        _pool_all(pl, lens)
        ids = torch.empty((S, k), dtype=torch.int32, device="cuda")
        cnt = torch.empty(S, dtype=torch.int32, device="cuda")
        sc = torch.zeros((S, L // 4), dtype=torch.float64, device="cuda")
        _topk_call(pl, dev(w.qI), pl.lens, S, L, k, ids, cnt, sc)
        out = torch.empty((S, HQ, D), dtype=torch.float32, device="cuda")
        _sparse_call(dev(w.q), pl.kv, pl.pg, ids, cnt, k, S, L, out)
        torch.cuda.synchronize()
        pooled = [O.read_pooled(pl.olay, pl.table_np, pl.arena_now(), s, L // 4) for s in range(S)]
        results.append([ids.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy(), out.cpu().numpy(),
                        np.stack(pooled)])
        del pl
        torch.cuda.empty_cache()
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
