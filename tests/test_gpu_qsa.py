"""GPU parity of block pooling, block scores + top-k, sparse attention and row
stores/gathers with the float64 oracle.

TensorFold PR #1169 "Receipt": for block scores, sparse attention rows, stores
and pooled rows, paged results match contiguous on each of three runs.  Pooled rows, scores
and top-k ids are compared bit for bit with the oracle (both sides use the same
float64 order); sparse attention rows within 2e-3 (max-norm relative a row).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import paged_kv_cache_pg_amd as P  # noqa: E402
from paged_kv_cache_pg_amd.inputs import make_workload, f32_to_bf16_bits  # noqa: E402
from gpu_util import Placed, decode, dev, rel_err_rows, TOL  # noqa: E402

HQ, HKV, DI, HI = 32, 4, 128, 4


def _qsa_workload(seed, lens, ptok, table_kind="shuffled"):
    return make_workload(seed, lens, ptok, HQ, HKV, dtype="bf16", table_kind=table_kind, idx_dim=DI, n_idx_heads=HI)


def _pool(pl, begin=None, end=None):
    w = pl.w
    S = w.n_streams
    b0 = dev(np.zeros(S, np.int32) if begin is None else np.array(begin, np.int32))
    b1 = dev(np.array([L // 4 for L in w.lens], np.int32) if end is None else np.array(end, np.int32))
    P.paged_pool_blocks(pl.ik, pl.pooled, DI, P.PAGED_BF16, pl.pg, b0, b1, S, max(w.lens))
    torch.cuda.synchronize()


def _pooled_gpu(pl):
    arena = pl.arena_now()
    return [O.read_pooled(pl.olay, pl.table_np, arena, s, L // 4) for s, L in enumerate(pl.w.lens)]


def _topk(pl, k, out_scores=True):
    w = pl.w
    S = w.n_streams
    max_len = max(w.lens)
    qi = dev(w.qI)
    ids = torch.full((S, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(S, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, max_len // 4), dtype=torch.float64, device="cuda") if out_scores else None
    ws = torch.empty(P.paged_topk_workspace(S, max_len, k), dtype=torch.uint8, device="cuda")
    P.paged_block_scores_topk(qi, P.PAGED_BF16, HI, DI, pl.pooled, P.PAGED_BF16, pl.pg, pl.lens, S, max_len, k,
                              ids, cnt, sc, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), cnt.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)


def _sparse(pl, ids, cnt, k, q=None):
    w = pl.w
    S = w.n_streams
    out = torch.empty((S, HQ, 256), dtype=torch.float32, device="cuda")
    ws = torch.zeros(P.paged_sparse_attn_workspace(S, HQ, k), dtype=torch.uint8, device="cuda")
    P.paged_sparse_attn(dev(w.q) if q is None else q, P.PAGED_BF16, HQ, pl.kv, pl.pg, dev(ids), dev(cnt), k, S,
                        max(w.lens), 1 / 16, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("ptok", [16, 48, 256])
def test_pool_bitwise_paged_and_contiguous(ptok):
    w = _qsa_workload(51, [1000, 517], ptok)
    want = O.pool(w.as_f64("IK"), w.lens)
    for paged in (True, False):
        pl = Placed(w, paged=paged)
        _pool(pl)
        got = _pooled_gpu(pl)
        for s in range(2):
            assert np.array_equal(got[s].view(np.uint32), want[s].view(np.uint32)), (paged, s)


def test_pool_incremental_equals_one_pass():
    """Blocks pooled in two calls (as a decode step completes them) give the same rows."""
    w = _qsa_workload(52, [800, 800], 48)
    pl = Placed(w)
    _pool(pl, [0, 0], [77, 3])
    _pool(pl, [77, 3], [200, 200])
    got = _pooled_gpu(pl)
    want = O.pool(w.as_f64("IK"), w.lens)
    for s in range(2):
        assert np.array_equal(got[s], want[s])


@pytest.mark.parametrize("k", [1, 37, 512, 4096])
def test_scores_and_topk_bitwise(k):
    w = _qsa_workload(53, [8192, 5000, 100], 256)
    pl = Placed(w)
    _pool(pl)
    ids, cnt, sc = _topk(pl, k)
    pooled = O.pool(w.as_f64("IK"), w.lens)
    qI = w.as_f64("qI")
    for s, L in enumerate(w.lens):
        want_sc = O.scores(qI[s], pooled[s])
        assert np.array_equal(sc[s, :L // 4].view(np.uint64), want_sc.view(np.uint64)), s
        want = O.topk(want_sc, k)
        n = len(want)
        assert cnt[s] == n
        assert np.array_equal(ids[s, :n], want), s
        assert np.all(ids[s, n:] == -1)


def test_topk_workspace_reused_over_shapes():
    """One workspace over calls of different shapes (a call with more streams than the one before puts
    its score histograms where the earlier call left selection data): the ids equal the oracle's every
    time."""
    cases = ((62, [20000], 300, 256), (61, [8000, 3000, 513], 64, 48), (63, [4000, 4000], 1000, 16),
             (64, [9000, 100, 7000], 200, 128))
    need = max(P.paged_topk_workspace(len(lens), max(lens), k) for _, lens, k, _ in cases)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    for seed, lens, k, ptok in cases:
        w = _qsa_workload(seed, lens, ptok)
        pl = Placed(w)
        _pool(pl)
        S, max_len = w.n_streams, max(w.lens)
        ids = torch.full((S, k), -7, dtype=torch.int32, device="cuda")
        cnt = torch.empty(S, dtype=torch.int32, device="cuda")
        P.paged_block_scores_topk(dev(w.qI), P.PAGED_BF16, HI, DI, pl.pooled, P.PAGED_BF16, pl.pg, pl.lens, S,
                                  max_len, k, ids, cnt, None, ws)
        torch.cuda.synchronize()
        pooled = O.pool(w.as_f64("IK"), w.lens)
        ids, cnt = ids.cpu().numpy(), cnt.cpu().numpy()
        for s in range(S):
            want = O.topk(O.scores(w.as_f64("qI")[s], pooled[s]), k)
            assert cnt[s] == len(want) and np.array_equal(ids[s, :len(want)], want), (seed, s)


def test_topk_exact_ties_lowest_id_wins():
    """Integer-valued indexer keys and queries in {-1, 0, 1}: scores tie exactly and often."""
    w = _qsa_workload(54, [4096, 4096, 2048], 128)
    rng = np.random.default_rng(7)
    w.IK = f32_to_bf16_bits(rng.integers(-1, 2, size=w.IK.shape).astype(np.float32))
    w.qI = f32_to_bf16_bits(rng.integers(-1, 2, size=w.qI.shape).astype(np.float32))
    pl = Placed(w)
    _pool(pl)
    ids, cnt, sc = _topk(pl, 300)
    pooled = O.pool(w.as_f64("IK"), w.lens)
    for s, L in enumerate(w.lens):
        want_sc = O.scores(w.as_f64("qI")[s], pooled[s])
        assert len(np.unique(want_sc)) < len(want_sc) // 4       # ties really happen
        assert np.array_equal(ids[s], O.topk(want_sc, 300))
    # all scores equal: the first k ids
    w.IK[:] = f32_to_bf16_bits(np.ones(1, np.float32))[0]
    pl = Placed(w)
    _pool(pl)
    ids, cnt, _ = _topk(pl, 100)
    for s in range(3):
        assert list(ids[s]) == list(range(100))


def test_sparse_matches_oracle_and_contiguous():
    w = _qsa_workload(55, [4096, 2000, 333], 48)
    pl, pc = Placed(w), Placed(w, paged=False)
    for p in (pl, pc):
        _pool(p)
    k = 64
    ids, cnt, _ = _topk(pl, k)
    ids_c, cnt_c, _ = _topk(pc, k)
    assert np.array_equal(ids, ids_c) and np.array_equal(cnt, cnt_c)
    outs = [_sparse(pl, ids, cnt, k) for _ in range(3)]
    oc = _sparse(pc, ids, cnt, k)
    for o in outs:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), oc.view(np.uint32))
    sel = [list(ids[s, :cnt[s]]) for s in range(3)]
    ref = O.sparse(w.as_f64("q"), w.as_f64("K"), w.as_f64("V"), sel, 1 / 16)
    assert rel_err_rows(outs[0], ref) <= TOL


def test_sparse_all_blocks_equals_dense_bitwise():
    """Every block selected, ascending: the same keys in the same order as dense decode."""
    w = _qsa_workload(56, [4096, 1024], 256)
    pl = Placed(w)
    k = 1024
    ids = np.full((2, k), -1, np.int32)
    cnt = np.zeros(2, np.int32)
    for s, L in enumerate(w.lens):
        ids[s, :L // 4] = np.arange(L // 4)
        cnt[s] = L // 4
    sp = _sparse(pl, ids, cnt, k)
    dn = decode(pl, dev(w.q), 1 / 16).cpu().numpy()
    assert np.array_equal(sp.view(np.uint32), dn.view(np.uint32))


def test_sparse_skips_out_of_range_ids():
    w = _qsa_workload(57, [512, 512], 16)
    pl = Placed(w)
    ids = np.array([[0, 5, 9999, 7], [3, -4, 2, 1]], np.int32)
    cnt = np.array([4, 4], np.int32)
    got = _sparse(pl, ids, cnt, 4)
    ref = O.sparse(w.as_f64("q"), w.as_f64("K"), w.as_f64("V"), [[0, 5, 7], [3, 2, 1]], 1 / 16)
    assert rel_err_rows(got, ref) <= TOL


def test_qsa_full_size_three_streams_131072():
    """3 streams x 131072 positions, pages of 256: pool, scores, top-512, sparse attention."""
    w = _qsa_workload(5, [131072] * 3, 256)
    pl = Placed(w)
    _pool(pl)
    k = 512
    ids, cnt, sc = _topk(pl, k)
    pooled = O.pool(w.as_f64("IK"), w.lens)
    qI = w.as_f64("qI")
    sel = []
    for s in range(3):
        want_sc = O.scores(qI[s], pooled[s])
        assert np.array_equal(sc[s].view(np.uint64), want_sc.view(np.uint64))
        want = O.topk(want_sc, k)
        assert np.array_equal(ids[s], want)
        sel.append(list(want))
    out = _sparse(pl, ids, cnt, k)
    qf = w.as_f64("q")
    for s in range(3):
        pos = np.array([4 * b + j for b in sel[s] for j in range(4)])
        Ks = (w.K[s:s + 1][:, :, pos].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        Vs = (w.V[s:s + 1][:, :, pos].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = O.decode(qf[s:s + 1], Ks, Vs, [len(pos)], 1 / 16)
        assert rel_err_rows(out[s:s + 1], ref) <= TOL


@pytest.mark.parametrize("ptok", [16, 48, 512])
def test_rows_store_and_gather_bitwise(ptok):
    """Rows stored through the table land where the oracle places them; a gather reads them back."""
    w = make_workload(58, [3000, 1234], ptok, 16, 4, dtype="bf16", table_kind="shuffled", idx_dim=DI, n_idx_heads=HI)
    olay = O.PageLayout(4, 256, ptok, "bf16", idx_dim=DI)
    lay = P.ArenaLayout(4, 256, ptok, P.PAGED_BF16, idx_dim=DI)
    want = O.place(olay, w.table, w.n_pages, w.lens, w.K, w.V, w.IK)
    arena = torch.zeros(len(want), dtype=torch.uint8, device="cuda")
    table = dev(w.table)
    pg = P.make_pg(table, ptok, lay.page_elems)
    lens = dev(np.array(w.lens, np.int32))
    zero = dev(np.zeros(2, np.int32))
    L = w.K.shape[2]
    Kd, Vd, IKd = dev(w.K), dev(w.V), dev(w.IK)
    base = arena.data_ptr()
    P.paged_rows_store(Kd, 4 * L * 256, L * 256, 256, base + lay.k_off, 4, 256, P.PAGED_BF16, pg, zero, lens, 2, L)
    P.paged_rows_store(Vd, 4 * L * 256, L * 256, 256, base + lay.v_off, 4, 256, P.PAGED_BF16, pg, zero, lens, 2, L)
    P.paged_rows_store(IKd, L * DI, 0, DI, base + lay.ik_off, 1, DI, P.PAGED_BF16, pg, zero, lens, 2, L)
    torch.cuda.synchronize()
    assert np.array_equal(arena.cpu().numpy(), want)
    back = torch.zeros_like(Kd)
    P.paged_rows_gather(back, 4 * L * 256, L * 256, 256, base + lay.k_off, 4, 256, P.PAGED_BF16, pg, zero, lens, 2, L)
    torch.cuda.synchronize()
    b = back.cpu().numpy().view(np.uint16)
    for s, Ls in enumerate(w.lens):
        assert np.array_equal(b[s, :, :Ls], w.K[s, :, :Ls])


def _topk_checked(w, pl, k, max_len=None):
    """Pool, then scores + top-k through the C ABI; scores and ids compared bit for bit with the oracle."""
    S = w.n_streams
    max_len = max_len or max(w.lens)
    b0 = dev(np.zeros(S, np.int32))
    b1 = dev(np.array([L // 4 for L in w.lens], np.int32))
    P.paged_pool_blocks(pl.ik, pl.pooled, w.idx_dim, P.PAGED_BF16, pl.pg, b0, b1, S, max_len)
    ids = torch.full((S, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(S, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, max_len // 4), dtype=torch.float64, device="cuda")
    ws = torch.empty(max(16, P.paged_topk_workspace(S, max_len, k)), dtype=torch.uint8, device="cuda")
    P.paged_block_scores_topk(dev(w.qI), P.PAGED_BF16, w.n_idx_heads, w.idx_dim, pl.pooled, P.PAGED_BF16, pl.pg,
                              pl.lens, S, max_len, k, ids, cnt, sc, ws)
    torch.cuda.synchronize()
    ids, cnt, sc = ids.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()
    pooled = O.pool(w.as_f64("IK"), w.lens)
    for s, L in enumerate(w.lens):
        want_sc = O.scores(w.as_f64("qI")[s], pooled[s])
        assert np.array_equal(sc[s, :L // 4].view(np.uint64), want_sc.view(np.uint64)), s
        want = O.topk(want_sc, k)
        assert cnt[s] == len(want)
        assert np.array_equal(ids[s, :len(want)], want), s
        assert np.all(ids[s, len(want):] == -1)


@pytest.mark.parametrize("di,hi", [(192, 3), (64, 2), (8, 1)])
def test_scores_other_indexer_widths(di, hi):
    """Indexer rows that are not 128 wide (staged in chunks of up to 128 dims)."""
    w = make_workload(59, [3000, 777], 48, 2, 1, dtype="bf16", table_kind="shuffled", idx_dim=di, n_idx_heads=hi)
    _topk_checked(w, Placed(w), 100)


def test_topk_more_blocks_than_the_register_path():
    """67,500 blocks in one stream: scores read from memory in every pass, ids compacted in two rounds."""
    w = make_workload(60, [270000, 1000], 256, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=128,
                      n_idx_heads=4)
    _topk_checked(w, Placed(w), 700)


def test_topk_register_path_bound_with_a_wide_table():
    """max_len just past the register path's 32,768 blocks while the streams are short."""
    w = make_workload(61, [9000, 4000], 256, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=128, n_idx_heads=4)
    stride = (131076 + 255) // 256
    table = np.zeros((2, stride), np.int32)
    table[:, :w.table.shape[1]] = w.table
    _topk_checked(w, Placed(w, table=table), 512, max_len=131076)


def test_topk_k_beyond_the_list_bound():
    """k = 9000 of 40,000 blocks: the taken ids go straight from the selection bits to the output."""
    w = make_workload(62, [160000, 30000], 256, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=128,
                      n_idx_heads=4)
    _topk_checked(w, Placed(w), 9000)


def test_topk_heavy_ties_take_the_radix_path():
    """More bin-T candidates than the ranking holds: every score equal over 5,000 and 4,250 blocks
    (the first k ids), then integer-valued keys over 10,000 blocks, both against the oracle."""
    w = make_workload(63, [20000, 17000], 64, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=128,
                      n_idx_heads=4)
    w.IK[:] = f32_to_bf16_bits(np.ones(1, np.float32))[0]
    _topk_checked(w, Placed(w), 700)
    w = make_workload(64, [40000], 64, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=128, n_idx_heads=4)
    rng = np.random.default_rng(8)
    w.IK = f32_to_bf16_bits(rng.integers(-1, 2, size=w.IK.shape).astype(np.float32))
    w.qI = f32_to_bf16_bits(rng.integers(-1, 2, size=w.qI.shape).astype(np.float32))
    _topk_checked(w, Placed(w), 300)


def test_topk_many_candidates_in_few_selection_workgroups():
    """Scores set block by block (indexer key = the block's value in dim 0, query = e0): 2,000 and
    1,500 blocks tied in 16 values inside one coarse bin, packed into two selection workgroups, so
    that they overflow the finishing workgroup's first gather and fill its sub-bins with ties."""
    lens = [32768, 30001]
    w = make_workload(65, lens, 256, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=128, n_idx_heads=4)
    rng = np.random.default_rng(9)
    v = np.zeros((2, 8192), np.float32)
    v[:] = rng.uniform(-1.0, 0.9, size=v.shape)
    v[0, :2000] = 1 + (np.arange(2000) % 16) / 128
    v[0, 2000:3000] = 2.0
    v[1, 6000:7500] = 1 + (np.arange(1500) * 7 % 16) / 128
    v[1, :500] = 2.0
    IK = np.zeros(w.IK.shape, np.float32)
    IK[:, :, 0] = np.repeat(v, 4, axis=1)[:, :IK.shape[1]]
    w.IK = f32_to_bf16_bits(IK)
    qI = np.zeros(w.qI.shape, np.float32)
    qI[:, 0, 0] = 1.0
    w.qI = f32_to_bf16_bits(qI)
    _topk_checked(w, Placed(w), 1500)
    _topk_checked(w, Placed(w), 1000)


@pytest.mark.parametrize("di,hi", [(128, 4), (128, 16), (64, 3)])
def test_scores_topk_float32_rows_and_queries(di, hi):
    """Float32 indexer keys and queries (the 128-wide kernel widens 16-byte query chunks; other
    widths take the staged kernel), pooled, scored and selected bit for bit against the oracle."""
    lens = [6000, 1001]
    w = make_workload(66, lens, 64, 2, 1, dtype="f32", table_kind="shuffled", idx_dim=di, n_idx_heads=hi)
    pl = Placed(w)
    S, ml, k = len(lens), max(lens), 200
    b0 = dev(np.zeros(S, np.int32))
    b1 = dev(np.array([L // 4 for L in lens], np.int32))
    P.paged_pool_blocks(pl.ik, pl.pooled, di, P.PAGED_F32, pl.pg, b0, b1, S, ml)
    ids = torch.full((S, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(S, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, ml // 4), dtype=torch.float64, device="cuda")
    ws = torch.empty(P.paged_topk_workspace(S, ml, k), dtype=torch.uint8, device="cuda")
    P.paged_block_scores_topk(dev(w.qI), P.PAGED_F32, hi, di, pl.pooled, P.PAGED_F32, pl.pg, pl.lens, S, ml, k,
                              ids, cnt, sc, ws)
    torch.cuda.synchronize()
    ids, cnt, sc = ids.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()
    pooled = O.pool(w.as_f64("IK"), lens)
    for s, L in enumerate(lens):
        want_sc = O.scores(w.as_f64("qI")[s], pooled[s])
        assert np.array_equal(sc[s, :L // 4].view(np.uint64), want_sc.view(np.uint64)), s
        want = O.topk(want_sc, k)
        assert cnt[s] == len(want)
        assert np.array_equal(ids[s, :len(want)], want), s


def test_topk_stream_past_the_selection_bitmap():
    """262,145 blocks in one stream (1,048,580 positions), one more than the finishing workgroup's
    bitmap holds: the single-workgroup list path selects, bit for bit against the oracle."""
    w = make_workload(67, [1048580], 256, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=128, n_idx_heads=1)
    _topk_checked(w, Placed(w), 512)


def test_scores_sum_order_matches_oracle():
    """Pooled rows and queries built so that the order of the float64 additions decides the score
    (2^60 absorbs a 1 added after it): the kernel must take the oracle's order -- queries summed over
    heads first, products in 8 groups by 4-dim chunk, each group in increasing dims, the groups
    meeting in the tree ((g0 + g1) + (g2 + g3)) + ((g4 + g5) + (g6 + g7)).  Six streams, each with one
    crafted row in every block, give 1, 0, 1, 0, 1, 0 in that order and other orders would not."""
    big = 2.0 ** 60
    lens = [64] * 6
    w = make_workload(68, lens, 16, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=128, n_idx_heads=3)
    rows = [{4: 1.0, 32: big, 33: -big},       # groups: g1 = 1, g0 = 0             -> 1
            {0: 1.0, 32: big, 33: -big},       # in-group order: (1 + 2^60) - 2^60   -> 0
            {0: 1.0, 8: big, 12: -big},        # tree pairs: (1 + 0) + (2^60 - 2^60) -> 1
            {0: big, 4: 1.0, 16: -big},        # halves: (2^60 + 1) + (-2^60)        -> 0
            {0: 1.0, 4: 1.0},                  # heads first (queries below)         -> 1
            {0: 1.0}]                          # heads in order (queries below)      -> 0
    IK = np.zeros(w.IK.shape, np.float32)
    for s, r in enumerate(rows):
        for d, x in r.items():
            IK[s, :, d] = x
    w.IK = f32_to_bf16_bits(IK)
    qI = np.zeros(w.qI.shape, np.float32)
    qI[:4, 0, :] = 1.0
    qI[4, 0, 0], qI[4, 1, 4], qI[4, 2, 4] = 1.0, big, -big
    qI[5, 0, 0], qI[5, 1, 0], qI[5, 2, 0] = big, 1.0, -big
    w.qI = f32_to_bf16_bits(qI)
    pl = Placed(w)
    S, ml, k = 6, 64, 4
    b0 = dev(np.zeros(S, np.int32))
    b1 = dev(np.array([L // 4 for L in lens], np.int32))
    P.paged_pool_blocks(pl.ik, pl.pooled, 128, P.PAGED_BF16, pl.pg, b0, b1, S, ml)
    ids = torch.empty((S, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(S, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, ml // 4), dtype=torch.float64, device="cuda")
    ws = torch.empty(P.paged_topk_workspace(S, ml, k), dtype=torch.uint8, device="cuda")
    P.paged_block_scores_topk(dev(w.qI), P.PAGED_BF16, 3, 128, pl.pooled, P.PAGED_BF16, pl.pg, pl.lens, S, ml, k,
                              ids, cnt, sc, ws)
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    for s, want in enumerate([1.0, 0.0, 1.0, 0.0, 1.0, 0.0]):
        assert np.all(sc[s] == want), (s, sc[s])
    pooled = O.pool(w.as_f64("IK"), lens)
    for s in range(S):
        assert np.array_equal(sc[s], O.scores(w.as_f64("qI")[s], pooled[s])), s
    # ties everywhere: the first k ids
    assert np.array_equal(ids.cpu().numpy(), np.tile(np.arange(k, dtype=np.int32), (S, 1)))


def test_pool_sums_in_float64_and_rounds_once():
    """Rows 1, 2^-24, 2^-24, 0 in dim 0 (and 2^20, 2^-20, -2^20, 2^-21 in dim 1): summed exactly and
    rounded once they pool to 0.25 + 2^-25 (and (2^-20 + 2^-21) / 4); rounding after each float32
    addition would give 0.25 (and 2^-21 / 4)."""
    w = make_workload(69, [16], 16, 1, 1, dtype="bf16", table_kind="shuffled", idx_dim=8, n_idx_heads=1)
    IK = np.zeros(w.IK.shape, np.float32)
    IK[0, 0:4, 0] = [1.0, 2.0 ** -24, 2.0 ** -24, 0.0]
    IK[0, 0:4, 1] = [2.0 ** 20, 2.0 ** -20, -(2.0 ** 20), 2.0 ** -21]
    w.IK = f32_to_bf16_bits(IK)
    pl = Placed(w)
    b0, b1 = dev(np.zeros(1, np.int32)), dev(np.array([4], np.int32))
    P.paged_pool_blocks(pl.ik, pl.pooled, 8, P.PAGED_BF16, pl.pg, b0, b1, 1, 16)
    torch.cuda.synchronize()
    got = _pooled_gpu(pl)[0]
    assert got[0, 0] == np.float32(0.25 + 2.0 ** -25) and got[0, 0] != np.float32(0.25)
    assert got[0, 1] == np.float32((2.0 ** -20 + 2.0 ** -21) / 4)
    assert np.array_equal(got.view(np.uint32), O.pool(w.as_f64("IK"), [16])[0].view(np.uint32))
