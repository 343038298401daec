"""Decode results must not depend on what the workspace held before the call, nor on how many calls
used it before, and every output row must be written (also for streams with no keys, into an output
that starts as NaN): the split partials live in the workspace and are merged by the combine step.

Bar: outputs bit for bit equal across workspace fills (zeros, 0xFF bytes, random bytes, one workspace
reused several times) and within 2e-3 of the float64 oracle.  Covers the vector-ALU decode (bf16 one
query), the sparse path and the MFMA decode (a window of two queries).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import paged_kv_cache_pg_amd as P  # noqa: E402
from paged_kv_cache_pg_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_workload  # noqa: E402
from gpu_util import Placed, dev, guarded_out, out_guards_intact, rel_err_rows, TOL  # noqa: E402

D = 256
# 16 splits, 1 split, no keys, a partial last tile, a few splits
LENS = [40960, 129, 0, 3000, 64 * 8 * 5 + 17]


def _fills(nbytes, seed):
    rng = np.random.default_rng(seed)
    yield "zeros", torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    yield "0xff", torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
    yield "random", dev(rng.integers(0, 256, nbytes, dtype=np.uint8))


def _check_all_equal(outs):
    ref = outs[0][1]
    for name, o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), ref.view(np.uint32)), name


def test_decode_merge_independent_of_workspace_contents():
    w = make_workload(301, LENS, 256, 32, 4, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    S, ml = len(LENS), max(LENS)
    q = dev(w.q)
    nbytes = P.paged_attn_decode_workspace(S, 32, ml)
    outs = []
    for name, ws in _fills(nbytes, 1):
        reps = 5 if name == "random" else 1
        for r in range(reps):
            buf, out = guarded_out((S, 32, D))
            P.paged_attn_decode(q, P.PAGED_BF16, 32, pl.kv, pl.pg, pl.lens, S, ml, 1 / 16, out, ws)
            torch.cuda.synchronize()
            assert out_guards_intact(buf)
            outs.append((f"{name} call {r}", out.cpu().numpy()))
    _check_all_equal(outs)
    got = outs[0][1]
    assert np.all(got[2] == 0)  # the stream with no keys
    ref = O.decode(w.as_f64("q"), w.as_f64("K"), w.as_f64("V"), LENS, 1 / 16)
    assert rel_err_rows(got, ref) <= TOL


def test_sparse_merge_independent_of_workspace_contents():
    lens = [8192, 4000, 0]
    w = make_workload(302, lens, 128, 16, 2, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    S, k = len(lens), 700
    rng = np.random.default_rng(5)
    ids = np.full((S, k), -1, np.int32)
    cnt = np.zeros(S, np.int32)
    for s, L in enumerate(lens):
        n = min(k, L // 4)
        ids[s, :n] = np.sort(rng.choice(L // 4, n, replace=False)) if n else []
        cnt[s] = n
    nbytes = P.paged_sparse_attn_workspace(S, 16, k)
    outs = []
    for name, ws in _fills(nbytes, 2):
        for r in range(3 if name == "0xff" else 1):
            buf, out = guarded_out((S, 16, D))
            P.paged_sparse_attn(dev(w.q), P.PAGED_BF16, 16, pl.kv, pl.pg, dev(ids), dev(cnt), k, S, max(lens), 1 / 16,
                                out, ws)
            torch.cuda.synchronize()
            assert out_guards_intact(buf)
            outs.append((f"{name} call {r}", out.cpu().numpy()))
    _check_all_equal(outs)
    got = outs[0][1]
    assert np.all(got[2] == 0)
    sel = [list(ids[s, :cnt[s]]) for s in range(S)]
    ref = O.sparse(w.as_f64("q"), w.as_f64("K"), w.as_f64("V"), sel, 1 / 16)
    assert rel_err_rows(got[:2], ref[:2]) <= TOL


def test_window_merge_independent_of_workspace_contents():
    W, hq, hkv = 2, 32, 4
    w = make_workload(303, LENS, 256, hq, hkv, dtype="bf16", table_kind="shuffled")
    pl = Placed(w)
    S, ml = len(LENS), max(LENS)
    rng = np.random.default_rng(6)
    qb = f32_to_bf16_bits(rng.standard_normal((S, W, hq, D), dtype=np.float32))
    q = dev(qb)
    nbytes = P.paged_attn_decode_window_workspace(S, hq, W, ml)
    outs = []
    for name, ws in _fills(nbytes, 3):
        for r in range(3 if name == "zeros" else 1):
            buf, out = guarded_out((S, W, hq, D))
            P.paged_attn_decode_window(q, P.PAGED_BF16, hq, W, pl.kv, pl.pg, pl.lens, S, ml, 1 / 16, out, ws)
            torch.cuda.synchronize()
            assert out_guards_intact(buf)
            outs.append((f"{name} call {r}", out.cpu().numpy()))
    _check_all_equal(outs)
    got = outs[0][1]
    assert np.all(got[2] == 0)
    ref = O.decode_window(bf16_bits_to_f32(qb).astype(np.float64), w.as_f64("K"), w.as_f64("V"), LENS, 1 / 16)
    assert rel_err_rows(got, ref) <= TOL
