"""The C ABI loads, exports every entry point its header declares, and refuses bad
arguments before anything is enqueued (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_pg_amd as P
from paged_kv_cache_pg_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")

FAKE = 1 << 20          # a 16-byte aligned address that is never dereferenced
MIS = FAKE + 4          # misaligned


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|int|size_t|const char \*)\s*(paged_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared()
    assert len(names) >= 13
    L = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B._SIGS), "binding and header disagree"


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises: there is no other path to fall back on."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libpagedattn.so"))
    with pytest.raises(RuntimeError, match="missing"):
        P.strerror(0)
    with pytest.raises(RuntimeError, match="missing"):
        P.paged_attn_decode_workspace(4, 32, 40960)


def test_strerror():
    assert P.strerror(0) == "ok"
    assert "workspace" in P.strerror(-3)
    assert P.strerror(-99) == "unknown status"


def _kv(**kw):
    d = dict(k=FAKE, v=FAKE, dtype=B.PAGED_BF16, n_kv_heads=4, head_dim=256)
    d.update(kw)
    return B.make_kv(d["k"], d["v"], d["dtype"], d["n_kv_heads"], d["head_dim"])


def _pg(table=FAKE, stride=160, ptok=256, pe=524288):
    return B.PgStruct(table, stride, ptok, pe, 0)


def _decode(q=FAKE, qd=B.PAGED_BF16, hq=32, kv=None, pg=None, lens=FAKE, S=4, max_len=40960, scale=0.0625,
            out=FAKE, ws=FAKE, wsb=None):
    kv = kv or _kv()
    pg = pg or _pg()
    if wsb is None:
        wsb = P.paged_attn_decode_workspace(S, hq, max_len)
    return B.lib().paged_attn_decode(q, qd, hq, ctypes.byref(kv), ctypes.byref(pg), lens, S, max_len, scale, out,
                                     ws, wsb, 0)


def test_decode_refusals():
    E, U, W = B.PAGED_EINVAL, B.PAGED_EUNSUPPORTED, B.PAGED_EWORKSPACE
    assert _decode(kv=_kv(head_dim=128)) == U
    assert _decode(hq=30) == E                      # Hq % Hkv != 0
    assert _decode(hq=64) == U                      # G = 16 not served
    assert _decode(qd=B.PAGED_F32) == U             # q and KV types differ
    assert _decode(qd=7) == E
    assert _decode(pg=_pg(stride=159)) == E         # table shorter than max_len (a short run)
    assert _decode(pg=_pg(table=0, ptok=40959)) == E  # no table: cap below max_len
    assert _decode(pg=_pg(ptok=0)) == E
    assert _decode(pg=_pg(pe=524288 - 1)) == E      # page not a multiple of 16 bytes / too small
    assert _decode(pg=_pg(pe=1024)) == E            # K region does not fit in a page
    assert _decode(q=MIS) == E
    assert _decode(q=0) == E
    assert _decode(out=MIS) == E
    assert _decode(lens=0) == E
    assert _decode(kv=_kv(k=MIS)) == E
    assert _decode(wsb=P.paged_attn_decode_workspace(4, 32, 40960) - 1) == W
    assert _decode(ws=0) == W
    assert _decode(ws=MIS) == W
    assert _decode(scale=float("nan")) == E
    assert _decode(max_len=-1) == E
    assert _decode(S=-1) == E
    assert _decode(S=0, q=0, out=0, lens=0, ws=0) == B.PAGED_OK   # nothing to do, nothing touched


def test_poisoned_structs_are_refused():
    kv = _kv()
    pg = _pg()
    pg.reserved = 0xAAAAAAAAAAAAAAAA - (1 << 64)
    assert _decode(pg=pg) == B.PAGED_EINVAL
    kv.reserved = -1431655766  # 0xAAAAAAAA
    assert _decode(kv=kv) == B.PAGED_EINVAL
    raw = (ctypes.c_uint8 * ctypes.sizeof(B.PgStruct))(*([0xAA] * ctypes.sizeof(B.PgStruct)))
    assert B.lib().paged_attn_decode(FAKE, 1, 32, ctypes.byref(_kv()), ctypes.cast(raw, ctypes.POINTER(B.PgStruct)),
                                     FAKE, 4, 40960, 0.0625, FAKE, FAKE, 1 << 30, 0) == B.PAGED_EINVAL


def test_workspace_sizes():
    # 4 streams x 32 heads x 16 splits x (256 + 2) floats
    assert P.paged_attn_decode_workspace(4, 32, 40960) == 4 * 32 * 16 * 258 * 4
    assert P.paged_attn_decode_workspace(1, 8, 300) == 1 * 8 * 1 * 258 * 4
    assert P.paged_attn_decode_workspace(0, 8, 300) == 0
    assert P.paged_sparse_attn_workspace(3, 32, 512) == 3 * 32 * 4 * 258 * 4
    # histograms, then per 1024 blocks: 2 counts, 32 words of taken bits, 1024 (u64 key, i32 id) pairs
    assert P.paged_topk_workspace(3, 131072, 512) == 3 * 4096 * 4 + 3 * 32 * (8 + 128 + 1024 * 12) + 3 * 32768 * 8


def test_sparse_pool_topk_refusals():
    E = B.PAGED_EINVAL
    kv, pg = _kv(), _pg(ptok=254, pe=4 * 254 * 256 * 2)
    L = B.lib()
    ws = P.paged_sparse_attn_workspace(3, 32, 512)
    # page size not a multiple of 4 (the pages' rule for n)
    assert L.paged_sparse_attn(FAKE, 1, 32, ctypes.byref(kv), ctypes.byref(_pg(ptok=254, stride=600)), FAKE, FAKE,
                               512, 3, 131072, 0.0625, FAKE, FAKE, ws, 0) == E
    assert L.paged_sparse_attn(FAKE, 1, 32, ctypes.byref(kv), ctypes.byref(_pg(stride=512)), FAKE, FAKE, 0, 3,
                               131072, 0.0625, FAKE, FAKE, ws, 0) == E           # k < 1
    assert L.paged_pool_blocks(FAKE, FAKE, 128, 1, ctypes.byref(pg), FAKE, FAKE, 3, 131072, 0) == E
    assert L.paged_pool_blocks(FAKE, FAKE, 100, 1, ctypes.byref(_pg(stride=512)), FAKE, FAKE, 3, 131072, 0) == E
    pg5 = _pg(stride=512, pe=573440)
    assert L.paged_pool_blocks(FAKE, MIS, 128, 1, ctypes.byref(pg5), FAKE, FAKE, 3, 131072, 0) == E
    wt = P.paged_topk_workspace(3, 131072, 512)
    assert L.paged_block_scores_topk(FAKE, 1, 4, 128, FAKE, 1, ctypes.byref(pg5), FAKE, 3, 131072, 0, FAKE, FAKE,
                                     0, FAKE, wt, 0) == E                            # k = 0
    assert L.paged_block_scores_topk(FAKE, 1, 32, 128, FAKE, 1, ctypes.byref(pg5), FAKE, 3, 131072, 512, FAKE,
                                     FAKE, 0, FAKE, wt, 0) == E                      # 32 x 128 > 2048
    assert L.paged_block_scores_topk(FAKE, 1, 1, 1028, FAKE, 1, ctypes.byref(pg5), FAKE, 3, 131072, 512, FAKE,
                                     FAKE, 0, FAKE, wt, 0) == E                      # rows past 1024 dims
    assert L.paged_block_scores_topk(FAKE, 1, 4, 128, FAKE, 1, ctypes.byref(pg5), FAKE, 3, 131072, 512, FAKE, FAKE,
                                     0, FAKE, wt - 8, 0) == B.PAGED_EWORKSPACE


def test_rows_and_offsets_refusals():
    E = B.PAGED_EINVAL
    L = B.lib()
    pg = _pg(stride=10, ptok=16, pe=4 * 16 * 256 * 2)
    assert L.paged_rows_store(FAKE, 0, 0, 256, FAKE, 4, 255, 1, ctypes.byref(pg), FAKE, FAKE, 1, 160, 0) == E
    assert L.paged_rows_store(FAKE, 0, 0, 4, FAKE, 4, 256, 1, ctypes.byref(pg), FAKE, FAKE, 1, 160, 0) == E
    assert L.paged_rows_store(FAKE, 0, 0, 256, FAKE, 9, 256, 1, ctypes.byref(pg), FAKE, FAKE, 1, 160, 0) == E
    assert L.paged_rows_store(FAKE, 0, 0, 256, FAKE, 4, 256, 1, ctypes.byref(pg), FAKE, FAKE, 1, 161, 0) == E
    assert L.paged_rows_gather(FAKE, 0, 0, 256, FAKE, 4, 256, 1, ctypes.byref(pg), 0, FAKE, 1, 160, 0) == E
    bad = _pg()
    bad.reserved = 1
    assert L.paged_row_offsets(ctypes.byref(bad), 1, 256, FAKE, FAKE, FAKE, FAKE, 10, 0) == E
    assert L.paged_row_offsets(ctypes.byref(_pg()), 1, 256, FAKE, FAKE, FAKE, FAKE, 0, 0) == B.PAGED_OK


def test_prefill_refusals():
    E, U = B.PAGED_EINVAL, B.PAGED_EUNSUPPORTED
    L = B.lib()
    kv = _kv()
    pg = _pg(stride=32)
    assert L.paged_attn_prefill(FAKE, 0, 2048, 6144, 32, ctypes.byref(_kv(dtype=0)), ctypes.byref(pg), 1, 0.0625,
                                FAKE, 0, 0, 0) == U
    assert L.paged_attn_prefill(FAKE, 1, 2048, 6145, 32, ctypes.byref(kv), ctypes.byref(pg), 1, 0.0625, FAKE, 0, 0,
                                0) == E     # table too short for q_pos0 + n_q
    assert L.paged_attn_prefill(FAKE, 1, -1, 0, 32, ctypes.byref(kv), ctypes.byref(pg), 1, 0.0625, FAKE, 0, 0, 0) == E
    assert L.paged_attn_prefill(MIS, 1, 2048, 0, 32, ctypes.byref(kv), ctypes.byref(pg), 1, 0.0625, FAKE, 0, 0,
                                0) == E


def test_fp8_refusals():
    E, U = B.PAGED_EINVAL, B.PAGED_EUNSUPPORTED
    L = B.lib()
    F8 = B.PAGED_FP8_E4M3

    def kv8(ks=FAKE, vs=FAKE):
        return B.make_kv(FAKE, FAKE, F8, 4, 256, ks, vs)

    pg8 = _pg(pe=4 * 256 * 256 * 2 + 2 * 4 * 256 * 4)       # e4m3 page: bytes
    assert _decode(kv=kv8(), pg=pg8, qd=B.PAGED_F32) == U   # e4m3 rows take bf16 queries
    assert _decode(kv=kv8(), pg=pg8, qd=F8) == E            # e4m3 is no query type
    assert _decode(kv=kv8(ks=0), pg=pg8) == E               # scale regions are required
    assert _decode(kv=kv8(vs=FAKE + 2), pg=pg8) == E        # and 4-byte aligned
    assert _decode(kv=kv8(), pg=_pg(pe=4 * 256 * 256 - 16)) == E   # codes of a page do not fit
    assert L.paged_attn_prefill(FAKE, 1, 16, 0, 32, ctypes.byref(kv8()), ctypes.byref(pg8), 1, 0.0625, FAKE, 0, 0,
                                0) == U
    # the e4m3 store keeps no indexer keys
    assert L.paged_kv_append(FAKE, FAKE, FAKE, 1, ctypes.byref(kv8()), FAKE, FAKE, 128, ctypes.byref(pg8), FAKE, 4,
                             40960, 0) == U
    # indexer-key, pooled and copied rows are never e4m3
    assert L.paged_pool_blocks(FAKE, FAKE, 128, F8, ctypes.byref(pg8), FAKE, FAKE, 3, 131072, 0) == E
    assert L.paged_rows_store(FAKE, 0, 0, 256, FAKE, 4, 256, F8, ctypes.byref(pg8), FAKE, FAKE, 1, 160, 0) == E


def test_window_refusals():
    U = B.PAGED_EUNSUPPORTED
    L = B.lib()

    def win(W, hq=32, dtype=B.PAGED_BF16, ws=FAKE):
        kv = B.make_kv(FAKE, FAKE, dtype, 4, 256)
        pg = _pg()
        wsb = P.paged_attn_decode_window_workspace(4, hq, W, 40960)
        return L.paged_attn_decode_window(FAKE, 1, hq, W, ctypes.byref(kv), ctypes.byref(pg), FAKE, 4, 40960, 0.0625,
                                          FAKE, ws, wsb, 0)
    assert win(3) == U                   # 3 queries x 8 heads > 16 columns
    assert win(5, hq=4) == U             # windows of at most 4
    assert win(2, dtype=B.PAGED_F32) == U
    assert win(0) == B.PAGED_EINVAL
    assert win(2, ws=0) == B.PAGED_EWORKSPACE
    # workspace rows scale with the window
    assert P.paged_attn_decode_window_workspace(4, 32, 2, 40960) == 2 * P.paged_attn_decode_workspace(4, 32, 40960)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more it exits with a message, before touching a device."""
    import subprocess
    import sys
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2, (argv, r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr
        assert r.stdout == ""


def test_noalloc_refusals_come_before_any_device_work():
    """The allocation-free decode refuses what paged_attn_decode refuses, and a request whose split
    partials would not fit its scratch (PAGED_ESCRATCH), before looking up any device memory."""
    kv, pg = _kv(), _pg()

    def call(hq=32, S=4, max_len=40960, q=FAKE):
        return B.lib().paged_attn_decode_noalloc(q, B.PAGED_BF16, hq, ctypes.byref(kv), ctypes.byref(pg), FAKE, S,
                                                 max_len, 0.0625, FAKE, 0)
    assert call(S=64) == B.PAGED_ESCRATCH          # the partials of 64 x 32 heads x 16 splits do not fit
    assert P.paged_attn_decode_workspace(64, 32, 40960) > B.NOALLOC_SCRATCH_BYTES
    assert P.paged_attn_decode_workspace(32, 32, 40960) <= B.NOALLOC_SCRATCH_BYTES
    assert call(hq=30) == B.PAGED_EINVAL
    assert call(q=MIS) == B.PAGED_EINVAL
    assert call(S=0) == B.PAGED_OK
    assert "scratch" in P.strerror(B.PAGED_ESCRATCH)
