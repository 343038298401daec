"""The library allocates nothing and records no memset, so its calls can be captured in a HIP graph:
pooling, scores + top-k, sparse attention and dense decode captured once and replayed several times,
with eager work and synchronisations between the replays; every replay must equal the eager results
bit for bit (ids, scores, attention rows)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_pg_amd as P  # noqa: E402
from paged_kv_cache_pg_amd.inputs import make_workload  # noqa: E402
from gpu_util import Placed, dev  # noqa: E402

HQ, HKV, DI, HI, K = 32, 4, 128, 4, 64


def test_graph_replays_equal_eager():
    lens = [4096, 3000, 517]
    w = make_workload(71, lens, 256, HQ, HKV, dtype="bf16", table_kind="shuffled", idx_dim=DI, n_idx_heads=HI)
    pl = Placed(w)
    S, ml = len(lens), max(lens)
    b0 = dev(np.zeros(S, np.int32))
    b1 = dev(np.array([L // 4 for L in lens], np.int32))
    q, qi = dev(w.q), dev(w.qI)
    ids = torch.empty((S, K), dtype=torch.int32, device="cuda")
    cnt = torch.empty(S, dtype=torch.int32, device="cuda")
    sc = torch.empty((S, ml // 4), dtype=torch.float64, device="cuda")
    tws = torch.empty(P.paged_topk_workspace(S, ml, K), dtype=torch.uint8, device="cuda")
    sws = torch.empty(P.paged_sparse_attn_workspace(S, HQ, K), dtype=torch.uint8, device="cuda")
    dws = torch.empty(P.paged_attn_decode_workspace(S, HQ, ml), dtype=torch.uint8, device="cuda")
    sp = torch.empty((S, HQ, 256), dtype=torch.float32, device="cuda")
    dn = torch.empty((S, HQ, 256), dtype=torch.float32, device="cuda")

    def step():
        P.paged_pool_blocks(pl.ik, pl.pooled, DI, P.PAGED_BF16, pl.pg, b0, b1, S, ml)
        P.paged_block_scores_topk(qi, P.PAGED_BF16, HI, DI, pl.pooled, P.PAGED_BF16, pl.pg, pl.lens, S, ml, K,
                                  ids, cnt, sc, tws)
        P.paged_sparse_attn(q, P.PAGED_BF16, HQ, pl.kv, pl.pg, ids, cnt, K, S, ml, 1 / 16, sp, sws)
        P.paged_attn_decode(q, P.PAGED_BF16, HQ, pl.kv, pl.pg, pl.lens, S, ml, 1 / 16, dn, dws)

    def snapshot():
        torch.cuda.synchronize()
        return [t.cpu().numpy().copy() for t in (ids, cnt, sc, sp, dn)]

    step()
    want = snapshot()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # a warm call on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        # outputs spoiled and eager work in between, so a replay that skipped a kernel would show
        for t in (ids, cnt, sp, dn):
            t.fill_(-1)
        sc.fill_(float("nan"))
        _ = (torch.ones(1 << 20, device="cuda") * rep).sum()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for a, b, name in zip(got, want, ("ids", "count", "scores", "sparse", "decode")):
            if name == "scores":  # a stream's scores past its own blocks are not written
                for si, L in enumerate(lens):
                    assert np.array_equal(a[si, :L // 4].view(np.uint8), b[si, :L // 4].view(np.uint8)), (rep, si)
            else:
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (rep, name)
