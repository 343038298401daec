"""Seeded random shapes through decode, the windowed decode and sparse attention: stream counts,
lengths (0 .. 6000, ragged), page sizes, q/KV head ratios, window sizes and row types drawn from
one generator, each case checked against the float64 oracle (2e-3, max-norm relative a row) and,
paged through a shuffled table, bit for bit against the same rows placed contiguously."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import paged_kv_cache_pg_amd as P  # noqa: E402
from paged_kv_cache_pg_amd.inputs import (  # noqa: E402
    bf16_bits_to_f32, draw_e4m3_codes, draw_row_scales, f32_to_bf16_bits, make_table, make_workload)
from gpu_util import DT, Placed, PlacedFp8, decode, decode_fp8, dev, rel_err_rows, TOL  # noqa: E402

D = 256
PTOKS = [16, 32, 48, 64, 128, 256, 512]
GROUPS = [(8, 8), (16, 8), (16, 4), (32, 4), (8, 1), (32, 8)]


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    S = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 6000, S)]
    if rng.random() < 0.3:
        lens[0] = int(rng.integers(0, 70))  # a short stream
    ptok = int(rng.choice(PTOKS))
    hq, hkv = GROUPS[int(rng.integers(len(GROUPS)))]
    return rng, S, lens, ptok, hq, hkv


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(seed):
    rng, S, lens, ptok, hq, hkv = _case(seed)
    dtype = "f32" if seed % 4 == 3 else "bf16"
    w = make_workload(2000 + seed, lens, ptok, hq, hkv, dtype=dtype, table_kind="shuffled")
    pl, pc = Placed(w), Placed(w, paged=False)
    q = dev(w.q)
    got = decode(pl, q, 1 / 16).cpu().numpy()
    oc = decode(pc, q, 1 / 16).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oc.view(np.uint32)), (S, lens, ptok, hq, hkv, dtype)
    ref = O.decode(w.as_f64("q"), w.as_f64("K"), w.as_f64("V"), lens, 1 / 16)
    assert rel_err_rows(got, ref) <= TOL, (S, lens, ptok, hq, hkv, dtype)


@pytest.mark.parametrize("seed", range(6))
def test_random_window(seed):
    rng, S, lens, ptok, hq, hkv = _case(100 + seed)
    G = hq // hkv
    W = int(rng.choice([w for w in (1, 2, 3, 4) if w * G <= 16]))
    w = make_workload(3000 + seed, lens, ptok, hq, hkv, dtype="bf16", table_kind="shuffled")
    qb = f32_to_bf16_bits(rng.standard_normal((S, W, hq, D), dtype=np.float32))
    q = dev(qb)
    outs = []
    for pl in (Placed(w), Placed(w, paged=False)):
        ml = max(lens)
        ws = torch.zeros(max(16, P.paged_attn_decode_window_workspace(S, hq, W, ml)), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((S, W, hq, D), dtype=torch.float32, device="cuda")
        P.paged_attn_decode_window(q, P.PAGED_BF16, hq, W, pl.kv, pl.pg, pl.lens, S, ml, 1 / 16, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), (S, lens, ptok, hq, hkv, W)
    ref = O.decode_window(bf16_bits_to_f32(qb).astype(np.float64), w.as_f64("K"), w.as_f64("V"), lens, 1 / 16)
    assert rel_err_rows(outs[0], ref) <= TOL, (S, lens, ptok, hq, hkv, W)


@pytest.mark.parametrize("seed", range(6))
def test_random_sparse(seed):
    rng, S, lens, ptok, hq, hkv = _case(200 + seed)
    w = make_workload(4000 + seed, lens, ptok, hq, hkv, dtype="bf16", table_kind="shuffled")
    k = int(rng.integers(1, 400))
    ids = np.full((S, k), -1, np.int32)
    cnt = np.zeros(S, np.int32)
    sel = []
    for s, L in enumerate(lens):
        n = min(k, L // 4)
        chosen = np.sort(rng.choice(L // 4, n, replace=False)) if n else np.zeros(0, np.int64)
        ids[s, :n] = chosen
        cnt[s] = n
        sel.append(list(chosen))
    outs = []
    # block lists need pages of whole blocks: the contiguous stream holds a multiple of 4 positions
    cap4 = (max(lens + [4]) + 3) // 4 * 4
    for pl in (Placed(w), Placed(w, paged=False, cap=cap4)):
        ws = torch.zeros(P.paged_sparse_attn_workspace(S, hq, k), dtype=torch.uint8, device="cuda")
        out = torch.empty((S, hq, D), dtype=torch.float32, device="cuda")
        P.paged_sparse_attn(dev(w.q), P.PAGED_BF16, hq, pl.kv, pl.pg, dev(ids), dev(cnt), k, S, max(lens + [4]),
                            1 / 16, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), (S, lens, ptok, hq, hkv, k)
    ref = O.sparse(w.as_f64("q"), w.as_f64("K"), w.as_f64("V"), sel, 1 / 16)
    assert rel_err_rows(outs[0], ref) <= TOL, (S, lens, ptok, hq, hkv, k)


@pytest.mark.parametrize("seed", range(4))
def test_random_decode_e4m3(seed):
    rng, S, lens, ptok, hq, hkv = _case(300 + seed)
    cap = max(lens + [1])
    KC, VC = draw_e4m3_codes(rng, (S, hkv, cap, D)), draw_e4m3_codes(rng, (S, hkv, cap, D))
    KS, VS = draw_row_scales(rng, (S, hkv, cap)), draw_row_scales(rng, (S, hkv, cap))
    qb = f32_to_bf16_bits(rng.standard_normal((S, hq, D), dtype=np.float32))
    table, n_pages = make_table("shuffled", [(L + ptok - 1) // ptok for L in lens], rng)
    pl = PlacedFp8(lens, hkv, ptok, KC, VC, KS, VS, table=table, n_pages=n_pages)
    pc = PlacedFp8(lens, hkv, ptok, KC, VC, KS, VS)
    q = dev(qb)
    got = decode_fp8(pl, q, hq, 1 / 16).cpu().numpy()
    oc = decode_fp8(pc, q, hq, 1 / 16).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oc.view(np.uint32)), (S, lens, ptok, hq, hkv)
    ref = O.decode(bf16_bits_to_f32(qb).astype(np.float64), O.e4m3_dequantize(KC, KS), O.e4m3_dequantize(VC, VS),
                   lens, 1 / 16)
    assert rel_err_rows(got, ref) <= TOL, (S, lens, ptok, hq, hkv)
