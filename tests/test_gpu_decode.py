"""GPU parity of dense decode (paged_attn_decode) with the float64 oracle.

Bar (TensorFold PR #1169 "Receipt"): paged and contiguous outputs agree bit for bit
on each of three runs, every attention row is within the float64 bound (here 2e-3
max-norm relative per row), guards and inputs are left untouched, and both red
controls (pages placed under one table but read through another; one placed row
overwritten) are caught.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import paged_kv_cache_pg_amd as P  # noqa: E402
from paged_kv_cache_pg_amd.inputs import make_workload  # noqa: E402
from gpu_util import DT, Placed, decode, dev, guarded_out, out_guards_intact, rel_err_rows, TOL  # noqa: E402


def _oracle(w, scale, streams=None):
    q, K, V = w.as_f64("q"), w.as_f64("K"), w.as_f64("V")
    return O.decode(q, K, V, w.lens, scale)


def _run_case(w, scale, repeats=3):
    pl = Placed(w, paged=True)
    pc = Placed(w, paged=False)
    q = dev(w.q)
    arena_before = pl.arena_np.copy()
    outs = []
    for _ in range(repeats):
        buf, out = guarded_out((w.n_streams, w.n_q_heads, w.head_dim))
        decode(pl, q, scale, out=out)
        torch.cuda.synchronize()
        assert out_guards_intact(buf), "output canaries overwritten"
        outs.append(out.cpu().numpy().copy())
    oc = decode(pc, q, scale).cpu().numpy()
    for o in outs:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), "repeat differs"
    assert np.array_equal(outs[0].view(np.uint32), oc.view(np.uint32)), "paged != contiguous"
    assert pl.guards_intact() and np.array_equal(pl.arena_now(), arena_before), "arena or guards changed"
    return pl, pc, q, outs[0]


def test_config1_fp32_reversed_table():
    """1 stream, 8 q / 2 KV heads, D 256, 300 positions, pages of 16 in a reversed table, fp32, scale 1/16."""
    w = make_workload(1, [300], 16, 8, 2, dtype="f32", table_kind="reversed")
    assert list(w.table[0]) == list(range(18, -1, -1))
    pl, pc, q, out = _run_case(w, 1 / 16)
    err = rel_err_rows(out, _oracle(w, 1 / 16))
    assert err <= TOL, err


LENS = [1, 17, 511, 4096, 8191, 9000]
PAGES = [16, 48, 128, 256, 512]


@pytest.mark.parametrize("ptok", PAGES)
@pytest.mark.parametrize("L", LENS)
def test_page_shape_sweep(L, ptok):
    """2 streams shuffled through one arena, 16 q / 4 KV heads, bf16."""
    w = make_workload(2, [L, L], ptok, 16, 4, dtype="bf16", table_kind="shuffled")
    pl, pc, q, out = _run_case(w, 1 / 16)
    err = rel_err_rows(out, _oracle(w, 1 / 16))
    assert err <= TOL, err


def test_mixed_pair_concurrent_equals_solo():
    """A long and a short stream in one batch give the bytes each gives alone (PR #2244's class of bug)."""
    w = make_workload(2, [9000, 17], 48, 16, 4, dtype="bf16", table_kind="shuffled")
    pl, pc, q, out = _run_case(w, 1 / 16)
    assert rel_err_rows(out, _oracle(w, 1 / 16)) <= TOL
    for s in range(2):
        # the same stream alone: its own table row, its own length, a batch of one
        table1 = pl.table[s:s + 1].contiguous()
        pg1 = P.make_pg(table1, w.page_pos, pl.lay.page_elems)
        ws = torch.zeros(P.paged_attn_decode_workspace(1, 16, w.lens[s]), dtype=torch.uint8, device="cuda")
        o1 = torch.empty((1, 16, 256), dtype=torch.float32, device="cuda")
        P.paged_attn_decode(q[s:s + 1].contiguous(), P.PAGED_BF16, 16, pl.kv, pg1, pl.lens[s:s + 1].contiguous(), 1,
                            w.lens[s], 1 / 16, o1, ws)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy()[0].view(np.uint32), out[s].view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_batch_split_in_two_launches_equals_each_stream_alone(dtype):
    """5 streams of 8192+ keys over 4 KV heads make 5 x 64 workgroups of 8 heads, one round (256 CUs)
    and a quarter: the first 3 streams run as one launch and the last 2 as a second launch whose heads
    are spread over 2 workgroups each (float32 rows: groups of 8 always run as two workgroups of 4).
    Every stream's output equals the stream decoded alone (itself a launch with the heads spread over
    4 workgroups), bit for bit, and the oracle within 2e-3.  The three launches also take the three
    load-hint choices (K and V nontemporal; V plain; both plain), which must not change a value."""
    lens = [8200, 9000, 8192, 12000, 8500]
    w = make_workload(12, lens, 256, 32, 4, dtype=dtype, table_kind="shuffled")
    pl = Placed(w, paged=True)
    q = dev(w.q)
    out = decode(pl, q, 1 / 16).cpu().numpy()
    assert rel_err_rows(out, _oracle(w, 1 / 16)) <= TOL
    for s in range(len(lens)):
        table1 = pl.table[s:s + 1].contiguous()
        pg1 = P.make_pg(table1, w.page_pos, pl.lay.page_elems)
        ws = torch.zeros(P.paged_attn_decode_workspace(1, 32, w.lens[s]), dtype=torch.uint8, device="cuda")
        o1 = torch.empty((1, 32, 256), dtype=torch.float32, device="cuda")
        P.paged_attn_decode(q[s:s + 1].contiguous(), DT[dtype], 32, pl.kv, pg1, pl.lens[s:s + 1].contiguous(), 1,
                            w.lens[s], 1 / 16, o1, ws)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy()[0].view(np.uint32), out[s].view(np.uint32)), s


def test_red_controls():
    """Reading placed pages through a different table, and overwriting one placed row, must each
    change the output."""
    w = make_workload(3, [600, 600], 16, 16, 4, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    q = dev(w.q)
    ref = decode(pl, q, 1 / 16).cpu().numpy()
    t = pl.table.clone()
    a, b = t[0, 3].item(), t[1, 5].item()
    t[0, 3], t[1, 5] = b, a
    pg2 = P.make_pg(t, w.page_pos, pl.lay.page_elems)
    ws = torch.zeros(P.paged_attn_decode_workspace(2, 16, 600), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(torch.from_numpy(ref)).cuda()
    P.paged_attn_decode(q, P.PAGED_BF16, 16, pl.kv, pg2, pl.lens, 2, 600, 1 / 16, o2, ws)
    assert not np.array_equal(o2.cpu().numpy(), ref)
    # planted row: flip one value row of stream 1 inside the arena
    off = O.row_offset(w.table, 16, pl.olay.page_elems, 1, 2, 100, 256) * 2 + pl.olay.v_off
    pl.buf[pl.guard + off: pl.guard + off + 512] = 0x3F
    o3 = decode(pl, q, 1 / 16).cpu().numpy()
    assert not np.array_equal(o3[1], ref[1]) and np.array_equal(o3[0], ref[0])


def test_zero_length_and_clamp():
    """A stream of length 0 gives zeros; lengths above max_len are clamped to it."""
    w = make_workload(4, [0, 70, 70], 16, 8, 2, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    q = dev(w.q)
    out = decode(pl, q, 0.0625).cpu().numpy()
    assert np.all(out[0] == 0)
    ref = _oracle(w, 0.0625)
    assert rel_err_rows(out[1:], ref[1:]) <= TOL
    lens_big = dev(np.array([0, 70, 5000], np.int32))
    out2 = decode(pl, q, 0.0625, lens=lens_big, max_len=70).cpu().numpy()
    assert np.array_equal(out2.view(np.uint32), out.view(np.uint32))


def test_single_key_returns_value_row_exactly():
    w = make_workload(5, [1, 1], 16, 8, 2, dtype="bf16", table_kind="shuffled")
    out = decode(Placed(w), dev(w.q), 0.0625).cpu().numpy()
    V = w.as_f64("V")
    for s in range(2):
        for h in range(8):
            assert np.array_equal(out[s, h].astype(np.float64), V[s, h // 4, 0])


def test_row_offsets_hook_bitwise():
    w = make_workload(6, [1000, 333], 48, 8, 2, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    rng = np.random.default_rng(0)
    n = 4096
    st = rng.integers(0, 2, n).astype(np.int32)
    hd = rng.integers(0, 2, n).astype(np.int32)
    ps = np.array([rng.integers(0, w.lens[s]) for s in st], np.int32)
    out = torch.empty(n, dtype=torch.int64, device="cuda")
    P.paged_row_offsets(pl.pg, 2, 256, dev(st), dev(hd), dev(ps), out, n)
    got = out.cpu().numpy()
    want = np.array([O.row_offset(w.table, 48, pl.olay.page_elems, int(s), int(h), int(p), 256)
                     for s, h, p in zip(st, hd, ps)])
    assert np.array_equal(got, want)


def _oracle_by_group(w, lens, scale=1 / 16):
    """The oracle's rows for every (stream, q head), one (stream, KV head) at a time so that only one
    group's rows are widened to float64 at once."""
    S, Hq, Hkv = w.n_streams, w.n_q_heads, w.n_kv_heads
    G = Hq // Hkv
    qf = w.as_f64("q")
    ref = np.zeros((S, Hq, w.head_dim))
    for s in range(S):
        for g in range(Hkv):
            L = int(lens[s])
            K = (w.K[s:s + 1, g:g + 1, :L].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            V = (w.V[s:s + 1, g:g + 1, :L].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            ref[s, g * G:(g + 1) * G] = O.decode(qf[s:s + 1, g * G:(g + 1) * G], K, V, [L], scale)[0]
    return ref


def test_batched_decode_full_size_every_row():
    """4 streams x 40960 positions, pages of 256 shuffled, 32 q / 4 KV heads, bf16 (the launch the
    benchmark times, five 64-key tiles a wave): paged == contiguous bit for bit, and every one of the
    128 (stream, head) rows within the bound of the oracle."""
    w = make_workload(3, [40960] * 4, 256, 32, 4, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    pc = Placed(w, paged=False)
    q = dev(w.q)
    o1 = decode(pl, q, 1 / 16).cpu().numpy()
    o2 = decode(pc, q, 1 / 16).cpu().numpy()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    del pl, pc
    ref = _oracle_by_group(w, w.lens)
    num = np.max(np.abs(o1 - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    assert np.all(num <= TOL * den), np.max(num / den)


@pytest.mark.parametrize("ptok", [48, 256])
def test_decode_four_and_more_tiles_a_wave_every_row(ptok):
    """Streams long enough that each wave runs 3 to 5 tiles (its four-slot key_at ring wraps), G = 8:
    lengths 40960, 32768, 24000 and 16500 over shuffled pages of 48 and 256: paged == contiguous bit
    for bit, and every row within the bound of the oracle."""
    lens = [40960, 32768, 24000, 16500]
    w = make_workload(31, lens, ptok, 32, 4, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    pc = Placed(w, paged=False)
    q = dev(w.q)
    o1 = decode(pl, q, 1 / 16).cpu().numpy()
    o2 = decode(pc, q, 1 / 16).cpu().numpy()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert pl.guards_intact()
    del pl, pc
    ref = _oracle_by_group(w, lens)
    assert rel_err_rows(o1, ref) <= TOL


def test_dense_decode_three_streams_131072_every_row():
    """Dense decode over the block-sparse workload's streams (3 x 131072 positions, pages of 256
    shuffled, 32 q / 4 KV heads, 16 tiles a wave), the launch the benchmark times for context: paged ==
    contiguous bit for bit, and every row within the bound of the oracle."""
    L = 131072
    w = make_workload(5, [L] * 3, 256, 32, 4, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    q = dev(w.q)
    o1 = decode(pl, q, 1 / 16).cpu().numpy()
    del pl
    pc = Placed(w, paged=False)
    o2 = decode(pc, q, 1 / 16).cpu().numpy()
    del pc
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    ref = _oracle_by_group(w, w.lens)
    assert rel_err_rows(o1, ref) <= TOL


def test_workspace_reuse_decode_and_sparse():
    """One workspace serves many calls (decode and sparse alike); repeats give the same bytes."""
    w = make_workload(7, [5000, 300, 9000], 48, 16, 4, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    q = dev(w.q)
    max_len = 9000
    ws = torch.full((P.paged_attn_decode_workspace(3, 16, max_len),), 0xAB, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(4):
        out = torch.empty((3, 16, 256), dtype=torch.float32, device="cuda")
        P.paged_attn_decode(q, P.PAGED_BF16, 16, pl.kv, pl.pg, pl.lens, 3, max_len, 1 / 16, out, ws)
        ids = dev(np.tile(np.arange(8, dtype=np.int32), (3, 1)))
        cnt = dev(np.array([8, 8, 8], np.int32))
        sp = torch.empty_like(out)
        P.paged_sparse_attn(q, P.PAGED_BF16, 16, pl.kv, pl.pg, ids, cnt, 8, 3, max_len, 1 / 16, sp, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    assert rel_err_rows(outs[0], _oracle(w, 1 / 16)) <= TOL


def test_workspace_reuse_with_changing_inputs():
    """Calls that share a workspace but read different queries and lengths each match their own oracle
    rows: the merge never reads a partial left by an earlier call."""
    w = make_workload(8, [4000, 4000], 48, 16, 4, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    rng = np.random.default_rng(3)
    from paged_kv_cache_pg_amd.inputs import f32_to_bf16_bits
    ws = torch.zeros(P.paged_attn_decode_workspace(2, 16, 4000), dtype=torch.uint8, device="cuda")
    K, V = w.as_f64("K"), w.as_f64("V")
    for it in range(6):
        qb = f32_to_bf16_bits(rng.standard_normal((2, 16, 256)).astype(np.float32))
        lens = [int(rng.integers(1, 4001)), int(rng.integers(1, 4001))]
        out = torch.empty((2, 16, 256), dtype=torch.float32, device="cuda")
        P.paged_attn_decode(dev(qb), P.PAGED_BF16, 16, pl.kv, pl.pg, dev(np.array(lens, np.int32)), 2, 4000, 1 / 16,
                            out, ws)
        torch.cuda.synchronize()
        qf = (qb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = O.decode(qf, K, V, lens, 1 / 16)
        assert rel_err_rows(out.cpu().numpy(), ref) <= TOL, (it, lens)


def test_tables_from_the_page_pool_after_churn():
    """Page tables built by the library's host pool while streams grow page by page, a transient
    stream takes and returns pages and runs are claimed from the top (fragmented tables): paged ==
    contiguous bit for bit and within the bound of the oracle."""
    ptok, lens = 48, [3000, 1500, 700]
    need = [(L + ptok - 1) // ptok for L in lens]
    n_pages = sum(need) + 40
    st = np.zeros(P.paged_pool_state_bytes(n_pages), np.uint8)
    P.paged_pool_init(st, n_pages)
    rng = np.random.default_rng(11)
    table = np.zeros((3, max(need)), np.int32)
    have = [0, 0, 0]
    one = np.zeros(8, np.int32)
    transient, runs = [], []
    while have != need:
        s = int(rng.integers(0, 3))
        if have[s] < need[s]:
            assert P.paged_pool_alloc(st, 1, one) == P.PAGED_OK
            table[s, have[s]] = one[0]
            have[s] += 1
        r = rng.random()
        if r < 0.3 and P.paged_pool_alloc(st, 2, one) == P.PAGED_OK:
            transient.extend(one[:2].tolist())
        elif r < 0.5 and transient:
            k = int(rng.integers(1, len(transient) + 1))
            give = transient[:k]
            transient = transient[k:]
            P.paged_pool_free(st, np.array(give[::-1], np.int32), len(give))
        elif r < 0.55:
            first = P.paged_pool_claim_run(st, 3)
            if first != P.PAGED_EFULL:
                runs.append(first)
    assert len(set(table[s, i] for s in range(3) for i in range(need[s]))) == sum(need)
    w = make_workload(12, lens, ptok, 16, 4, dtype="bf16", table_kind="shuffled")
    w.table, w.n_pages = table, n_pages
    pl, pc, q, out = _run_case(w, 1 / 16)
    err = rel_err_rows(out, _oracle(w, 1 / 16))
    assert err <= TOL, err


@pytest.mark.parametrize("hq,hkv", [(32, 4), (16, 4), (8, 4), (4, 4)])
def test_bytes_independent_of_max_len(hq, hkv):
    """Short key lists spread a KV head's q heads over several workgroups; a head's arithmetic is the
    same either way, so a stream gives the same bytes with max_len = its own length (short path)
    and with max_len = 20000 (long path, one workgroup a KV head), and the sparse call over all of
    its blocks (k = 1024, short) equals the dense call with max_len = 20000 bit for bit."""
    lens = [4096, 777]
    w = make_workload(41, lens, 256, hq, hkv, dtype="bf16", table_kind="shuffled")
    big = 20000
    table = np.zeros((2, (big + 255) // 256), np.int32)
    table[:, :w.table.shape[1]] = w.table
    pl = Placed(w, table=table)
    q = dev(w.q)
    o_short = decode(pl, q, 1 / 16, max_len=max(lens)).cpu().numpy()
    o_long = decode(pl, q, 1 / 16, max_len=big).cpu().numpy()
    assert np.array_equal(o_short.view(np.uint32), o_long.view(np.uint32))
    assert rel_err_rows(o_short, _oracle(w, 1 / 16)) <= TOL
    k = 1024
    ids = np.full((2, k), -1, np.int32)
    cnt = np.zeros(2, np.int32)
    for s, L in enumerate(lens):
        ids[s, :L // 4] = np.arange(L // 4)
        cnt[s] = L // 4
    ws = torch.zeros(P.paged_sparse_attn_workspace(2, hq, k), dtype=torch.uint8, device="cuda")
    sp = torch.empty((2, hq, 256), dtype=torch.float32, device="cuda")
    P.paged_sparse_attn(q, P.PAGED_BF16, hq, pl.kv, pl.pg, dev(ids), dev(cnt), k, 2, big, 1 / 16, sp, ws)
    torch.cuda.synchronize()
    sp = sp.cpu().numpy()
    # stream 1 (777 positions) has a ragged last block the block list cannot name: compare stream 0
    assert np.array_equal(sp[0].view(np.uint32), o_long[0].view(np.uint32))
