"""GPU parity of chunked causal prefill (paged_attn_prefill, MFMA) with the float64 oracle.

A chunk of queries at positions q_pos0 .. q_pos0+n_q-1 attends, head by head, to the cached
keys 0 .. p (causal mask: key <= query position); the chunk's own rows are stored
before it runs.  Checks: paged == contiguous bit for bit, repeats bit for bit, rows within
2e-3 (max-norm relative a row) of the oracle, position 0 equal to the first value row.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import paged_kv_cache_pg_amd as P  # noqa: E402
from paged_kv_cache_pg_amd.inputs import make_workload  # noqa: E402
from gpu_util import Placed, dev, guarded_out, out_guards_intact, rel_err_rows, TOL  # noqa: E402


def _prefill(pl, q, n_q, q_pos0, causal=True, scale=1 / 16, out=None):
    w = pl.w
    if out is None:
        out = torch.empty((n_q, w.n_q_heads, 256), dtype=torch.float32, device="cuda")
    P.paged_attn_prefill(q, P.PAGED_BF16, n_q, q_pos0, w.n_q_heads, pl.kv, pl.pg, causal, scale, out)
    torch.cuda.synchronize()
    return out


def _case(seed, q_pos0, n_q, ptok, hq, hkv, table_kind="shuffled", causal=True, rows=None, check_oracle=True):
    kv_len = q_pos0 + n_q
    w = make_workload(seed, [kv_len], ptok, hq, hkv, dtype="bf16", table_kind=table_kind, n_queries=n_q)
    pl, pc = Placed(w), Placed(w, paged=False)
    q = dev(w.q)
    buf, out = guarded_out((n_q, hq, 256))
    _prefill(pl, q, n_q, q_pos0, causal, out=out)
    assert out_guards_intact(buf)
    o1 = out.cpu().numpy()
    o2 = _prefill(pl, q, n_q, q_pos0, causal).cpu().numpy()
    oc = _prefill(pc, q, n_q, q_pos0, causal).cpu().numpy()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), "repeat differs"
    assert np.array_equal(o1.view(np.uint32), oc.view(np.uint32)), "paged != contiguous"
    if check_oracle:
        ref = O.prefill(w.as_f64("q"), w.as_f64("K")[0], w.as_f64("V")[0], q_pos0, 1 / 16, causal=causal, rows=rows)
        sel = np.arange(n_q) if rows is None else np.asarray(rows)
        err = rel_err_rows(o1[sel], ref[sel])
        assert err <= TOL, err
    return w, o1


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (8, 2), (32, 4)])
def test_prefill_from_position_zero(hq, hkv):
    w, out = _case(11, 0, 100, 16, hq, hkv, table_kind="reversed")
    V = w.as_f64("V")[0]
    G = hq // hkv
    for h in range(hq):
        assert np.array_equal(out[0, h].astype(np.float64), V[h // G, 0])   # position 0 sees only key 0


@pytest.mark.parametrize("q_pos0,n_q,ptok", [(130, 77, 48), (2048, 200, 256), (5, 1, 16), (63, 130, 128)])
def test_prefill_chunk_ragged(q_pos0, n_q, ptok):
    _case(12, q_pos0, n_q, ptok, 32, 4)


def test_prefill_not_causal():
    _case(13, 300, 90, 48, 16, 4, causal=False)


def test_prefill_last_row_equals_decode():
    """The last query of a chunk attends to every cached key: its rows match decode over q_pos0 + n_q keys."""
    q_pos0, n_q = 1000, 24
    w, out = _case(14, q_pos0, n_q, 48, 16, 4)
    pl = Placed(w)
    L = q_pos0 + n_q
    qd = dev(np.ascontiguousarray(w.q[n_q - 1:n_q]))
    ws = torch.zeros(P.paged_attn_decode_workspace(1, 16, L), dtype=torch.uint8, device="cuda")
    dec = torch.empty((1, 16, 256), dtype=torch.float32, device="cuda")
    P.paged_attn_decode(qd, P.PAGED_BF16, 16, pl.kv, pl.pg, dev(np.array([L], np.int32)), 1, L, 1 / 16, dec, ws)
    torch.cuda.synchronize()
    assert rel_err_rows(out[n_q - 1], dec.cpu().numpy()[0]) <= 2 * TOL


def test_prefill_8192_in_chunks_of_2048_sampled():
    """One stream, 8192-token prompt as four 2048-query chunks over pages of 256 (shuffled),
    32 q / 4 KV heads: each chunk paged == contiguous bit for bit; sampled rows against the oracle."""
    w = make_workload(4, [8192], 256, 32, 4, dtype="bf16", table_kind="shuffled", n_queries=8192)
    pl, pc = Placed(w), Placed(w, paged=False)
    Kf, Vf = w.as_f64("K")[0], w.as_f64("V")[0]
    rng = np.random.default_rng(0)
    for c0 in range(0, 8192, 2048):
        qc = np.ascontiguousarray(w.q[c0:c0 + 2048])
        q = dev(qc)
        o1 = _prefill(pl, q, 2048, c0).cpu().numpy()
        oc = _prefill(pc, q, 2048, c0).cpu().numpy()
        assert np.array_equal(o1.view(np.uint32), oc.view(np.uint32))
        rows = np.unique(np.concatenate([[0, 1, 15, 16, 2047], rng.integers(0, 2048, 24)]))
        qf = (qc.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = O.prefill(qf, Kf, Vf, c0, 1 / 16, rows=rows)
        assert rel_err_rows(o1[rows], ref[rows]) <= TOL, c0


def test_prefill_40960_in_chunks_of_2048():
    """The 40960-token prompt (160 shuffled pages of 256, 32 q / 4 KV heads) as twenty 2048-query
    chunks, the launches the benchmark times: every chunk paged == contiguous bit for bit.  In the
    first and the last chunk, one query of every 16-query block (the queries of one workgroup), at a
    rotating place inside the block so that every wave's rows come up, is checked on all 32 heads
    against the oracle: every workgroup of those launches is covered.  A middle chunk is sampled."""
    n = 40960
    w = make_workload(4, [n], 256, 32, 4, dtype="bf16", table_kind="shuffled", n_queries=n)
    pl, pc = Placed(w), Placed(w, paged=False)
    Kf, Vf = w.as_f64("K")[0], w.as_f64("V")[0]
    rng = np.random.default_rng(1)
    per_block = np.arange(0, 2048, 16) + (np.arange(128) % 16)
    for c0 in range(0, n, 2048):
        qc = np.ascontiguousarray(w.q[c0:c0 + 2048])
        q = dev(qc)
        o1 = _prefill(pl, q, 2048, c0).cpu().numpy()
        oc = _prefill(pc, q, 2048, c0).cpu().numpy()
        assert np.array_equal(o1.view(np.uint32), oc.view(np.uint32)), c0
        assert np.isfinite(o1).all(), c0
        if c0 in (0, n - 2048):
            rows = per_block
        elif c0 == 20480:
            rows = np.unique(np.concatenate([[0, 2047], rng.integers(0, 2048, 6)]))
        else:
            continue
        qf = (qc.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = O.prefill(qf, Kf, Vf, c0, 1 / 16, rows=rows)
        assert rel_err_rows(o1[rows], ref[rows]) <= TOL, c0
