#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one batched paged decode: 4 streams x 40960 cached positions, pages of
256 positions in one shuffled arena, 32 query / 4 KV heads, head dim 256, bf16
K/V and q, fp32 accumulation, one query token a stream.  ``value`` is the
decode's algorithmic HBM bytes (K/V rows, q, table, lengths, output) over its
measured time, in GB/s.  The line also carries the roofline of the decode,
the float64 oracle timed on the host cores, and the other rows of the path
(chunked prefill, block pooling, scores + top-k, sparse attention, the
appends of a decode step and a prefill chunk) as extra objects.  Inputs are
seeded synthetic N(0, 1) draws; they sit in HBM before timing starts.  Two copies of the arena alternate between steps so the
256 MB Infinity Cache cannot serve a step from the previous one.

The oracle leg -- the float64 oracle timed on the host cores (``cpu_baseline``) and the spot checks
of sampled output rows against it, all outside the timed regions -- is the only part of this file
that runs anything under ``oracle/``; ``--no-cpu-baseline`` turns the whole leg off.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ORACLE_LEG = True  # cpu_baseline timings and the oracle spot checks; off with --no-cpu-baseline
MFMA_BF16_PEAK_TFLOPS = 2500.0

# HBM bytes per decode launch (split + combine) from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled
# by the same counters on a copy of known size (profiles/decode_4x40960_p256_hbm_traffic.md); valid
# only for the kernel sources that were measured.
DECODE_TRAFFIC_BYTES = 676_356_870
DECODE_TRAFFIC_SOURCES = "9be177aa5ee9f53a"
# The same for the e4m3 decode (MFMA kernel + combine; profiles/decode_e4m3_4x40960_p256.md).
FP8_TRAFFIC_BYTES = 345_900_367
FP8_TRAFFIC_SOURCES = "69f3b43ab22f404b"

_DECODE_SOURCES = ("paged_kv_cache_pg_amd/csrc/decode.hip", "paged_kv_cache_pg_amd/csrc/split.h",
                   "paged_kv_cache_pg_amd/csrc/common.h")
_FP8_SOURCES = ("paged_kv_cache_pg_amd/csrc/decode_mfma.hip", "paged_kv_cache_pg_amd/csrc/decode.hip",
                "paged_kv_cache_pg_amd/csrc/split.h", "paged_kv_cache_pg_amd/csrc/mfma.h",
                "paged_kv_cache_pg_amd/csrc/common.h")


def _sources_hash(files=_DECODE_SOURCES) -> str:
    """Hash of the kernels' code: comments dropped and whitespace collapsed, so that only a change
    to the code itself invalidates a traffic figure."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _decode_sources_hash() -> str:
    return _sources_hash(_DECODE_SOURCES)


def _err(x) -> str:
    return "(no oracle check)" if x is None else f"{x:.2e}"


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def _blas_threads() -> int:
    try:
        import threadpoolctl
        n = [i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def _affinity_cores() -> int:
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def _oracle_threads() -> dict:
    """What the host oracle ran on: the BLAS threads its matrix products used (the rest of it is one
    Python thread) and the cores the process may use."""
    return {"cores": _blas_threads(), "affinity_cores": _affinity_cores()}


# ---------------------------------------------------------------------------
# Batched paged decode (the headline)
# ---------------------------------------------------------------------------

class DecodeBench:
    S, L, PTOK, HQ, HKV, D = 4, 40960, 256, 32, 4, 256

    def __init__(self, seed: int = 3):
        import numpy as np
        import torch
        import paged_kv_cache_pg_amd as P
        from paged_kv_cache_pg_amd.inputs import make_workload

        self.P, self.torch, self.np = P, torch, np
        t0 = time.time()
        w = make_workload(seed, [self.L] * self.S, self.PTOK, self.HQ, self.HKV, dtype="bf16", table_kind="shuffled")
        self.w = w
        log(f"decode: workload drawn in {time.time() - t0:.1f}s")
        self.lay = P.ArenaLayout(self.HKV, self.D, self.PTOK, P.PAGED_BF16)
        self.table = torch.from_numpy(w.table.astype(np.int32)).cuda()
        self.pg = P.make_pg(self.table, self.PTOK, self.lay.page_elems)
        self.q = torch.from_numpy(w.q.view(np.int16)).cuda()
        self.lens = torch.tensor(w.lens, dtype=torch.int32, device="cuda")
        begin = torch.zeros(self.S, dtype=torch.int32, device="cuda")
        # place the rows with the library's own store kernel, through the table
        self.arenas = []
        for copy in range(2):
            arena = torch.zeros(w.n_pages * self.lay.page_bytes, dtype=torch.uint8, device="cuda")
            for name, off in (("K", self.lay.k_off), ("V", self.lay.v_off)):
                src = torch.from_numpy(getattr(w, name).view(np.int16)).cuda()
                P.paged_rows_store(src, self.HKV * self.L * self.D, self.L * self.D, self.D, arena.data_ptr() + off,
                                   self.HKV, self.D, P.PAGED_BF16, self.pg, begin, self.lens, self.S, self.L)
                torch.cuda.synchronize()
                del src
            self.arenas.append(arena)
        self.kvs = [P.make_kv(a.data_ptr() + self.lay.k_off, a.data_ptr() + self.lay.v_off, P.PAGED_BF16, self.HKV,
                              self.D) for a in self.arenas]
        self.ws = torch.zeros(P.paged_attn_decode_workspace(self.S, self.HQ, self.L), dtype=torch.uint8,
                              device="cuda")
        self.out = torch.empty((self.S, self.HQ, self.D), dtype=torch.float32, device="cuda")
        self.alg_bytes = (self.S * self.HKV * self.L * self.D * 2 * 2    # K and V rows
                          + self.q.numel() * 2                            # q
                          + self.S * w.table.shape[1] * 4                 # page table
                          + self.S * 4                                    # lengths
                          + self.out.numel() * 4)                         # output

    def step(self, i: int):
        self.P.paged_attn_decode(self.q, self.P.PAGED_BF16, self.HQ, self.kvs[i & 1], self.pg, self.lens, self.S,
                                 self.L, 1 / 16, self.out, self.ws)

    def check(self):
        """Sampled rows against the oracle (outside the timed region)."""
        import oracle as O
        np = self.np
        self.step(0)
        self.torch.cuda.synchronize()
        out = self.out.cpu().numpy()
        w = self.w
        qf, K, V = w.as_f64("q"), w.as_f64("K"), w.as_f64("V")
        worst = 0.0
        for s, h in [(0, 0), (3, 31)]:
            g = h // 8
            ref = O.decode(qf[s:s + 1, h:h + 1], K[s:s + 1, g:g + 1], V[s:s + 1, g:g + 1], [self.L], 1 / 16)[0, 0]
            worst = max(worst, float(np.max(np.abs(out[s, h] - ref)) / np.max(np.abs(ref))))
        return worst

    @classmethod
    def cpu_baseline_from_scratch(cls, seed: int = 3, min_seconds: float = 10.0):
        """The oracle (gather through the table + float64 attention) on the whole decode workload, drawn
        again on the host, repeated until at least ``min_seconds`` of CPU work have been timed."""
        import oracle as O
        from paged_kv_cache_pg_amd.inputs import bf16_bits_to_f32, make_workload
        w = make_workload(seed, [cls.L] * cls.S, cls.PTOK, cls.HQ, cls.HKV, dtype="bf16", table_kind="shuffled")
        olay = O.PageLayout(cls.HKV, cls.D, cls.PTOK, "bf16")
        arena = O.place(olay, w.table, w.n_pages, w.lens, w.K, w.V)
        qf = w.as_f64("q")
        reps, total = 0, 0.0
        while total < min_seconds:
            t0 = time.perf_counter()
            K, V, _ = O.gather(olay, w.table, arena, w.lens)
            K = bf16_bits_to_f32(K).astype("float64")
            V = bf16_bits_to_f32(V).astype("float64")
            O.decode(qf, K, V, w.lens, 1 / 16)
            total += time.perf_counter() - t0
            reps += 1
            del K, V
        kv_bytes = cls.S * cls.HKV * cls.L * cls.D * 2 * 2
        return {"value": round(reps * kv_bytes / total / 1e9, 4), "unit": "GB/s", **_oracle_threads(),
                "kind": "oracle",
                "sample": f"whole decode workload (4 streams x 40960 positions, 32 q / 4 KV heads): gather through "
                          f"the table + float64 attention, {reps} passes in {total:.2f} s"}


# ---------------------------------------------------------------------------
# Chunked causal prefill (MFMA)
# ---------------------------------------------------------------------------

class PrefillBench:
    """One stream, a prompt of N tokens processed as chunks of 2048 queries against its paged cache
    (pages of 256 shuffled), 32 q / 4 KV heads, head dim 256, bf16; all K/V rows stored first."""
    HQ, HKV, D, PTOK, CHUNK = 32, 4, 256, 256, 2048

    def __init__(self, n_tokens: int, seed: int = 4):
        import numpy as np
        import torch
        import paged_kv_cache_pg_amd as P
        from paged_kv_cache_pg_amd.inputs import make_workload
        self.P, self.torch, self.N = P, torch, n_tokens
        t0 = time.time()
        w = make_workload(seed, [n_tokens], self.PTOK, self.HQ, self.HKV, dtype="bf16", table_kind="shuffled",
                          n_queries=n_tokens)
        self.w = w
        log(f"prefill {n_tokens}: workload drawn in {time.time() - t0:.1f}s")
        lay = P.ArenaLayout(self.HKV, self.D, self.PTOK, P.PAGED_BF16)
        self.table = torch.from_numpy(w.table.astype(np.int32)).cuda()
        self.pg = P.make_pg(self.table, self.PTOK, lay.page_elems)
        lens = torch.tensor([n_tokens], dtype=torch.int32, device="cuda")
        begin = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.arena = torch.zeros(w.n_pages * lay.page_bytes, dtype=torch.uint8, device="cuda")
        for name, off in (("K", lay.k_off), ("V", lay.v_off)):
            src = torch.from_numpy(getattr(w, name).view(np.int16)).cuda()
            P.paged_rows_store(src, self.HKV * n_tokens * self.D, n_tokens * self.D, self.D,
                               self.arena.data_ptr() + off, self.HKV, self.D, P.PAGED_BF16, self.pg, begin, lens, 1,
                               n_tokens)
            torch.cuda.synchronize()
            del src
        self.kv = P.make_kv(self.arena.data_ptr() + lay.k_off, self.arena.data_ptr() + lay.v_off, P.PAGED_BF16,
                            self.HKV, self.D)
        self.q = torch.from_numpy(w.q.view(np.int16)).cuda()          # [N][Hq][D]
        self.out = torch.empty((self.CHUNK, self.HQ, self.D), dtype=torch.float32, device="cuda")
        self.flops = 4.0 * self.D * self.HQ * n_tokens * (n_tokens + 1) / 2   # unmasked QK^T + PV

    def chunk(self, c0: int):
        n = min(self.CHUNK, self.N - c0)
        self.P.paged_attn_prefill(self.q[c0:c0 + n], self.P.PAGED_BF16, n, c0, self.HQ, self.kv, self.pg, True,
                                  1 / 16, self.out)

    def run(self, i: int = 0):
        for c0 in range(0, self.N, self.CHUNK):
            self.chunk(c0)

    def oracle_rate(self, every: int = 4):
        """The oracle's prompt throughput, from a bounded sample: every `every`-th query of the last two
        chunks, all heads (those rows see almost the whole cache, so the oracle's work a row is the
        algorithmic one), gathered through the table and attended in float64; the FLOP rate of the
        sample is applied to the whole prompt's algorithmic FLOP."""
        import numpy as np
        import oracle as O
        from paged_kv_cache_pg_amd.inputs import bf16_bits_to_f32
        w = self.w
        olay = O.PageLayout(self.HKV, self.D, self.PTOK, "bf16")
        arena = O.place(olay, w.table, w.n_pages, w.lens, w.K, w.V)
        flops, t_total, rows_done = 0.0, 0.0, 0
        t0 = time.perf_counter()
        K, V, _ = O.gather(olay, w.table, arena, w.lens)
        Kf = bf16_bits_to_f32(K[0]).astype(np.float64)
        Vf = bf16_bits_to_f32(V[0]).astype(np.float64)
        t_total += time.perf_counter() - t0
        del K, V, arena
        for c0 in (self.N - 2 * self.CHUNK, self.N - self.CHUNK):
            qc = np.ascontiguousarray(w.q[c0:c0 + self.CHUNK])
            qf = bf16_bits_to_f32(qc).astype(np.float64)
            rows = np.arange(0, self.CHUNK, every)
            t0 = time.perf_counter()
            O.prefill(qf, Kf, Vf, c0, 1 / 16, rows=rows)
            t_total += time.perf_counter() - t0
            flops += 4.0 * self.D * self.HQ * float(np.sum(c0 + rows + 1))
            rows_done += len(rows)
        rate = flops / t_total
        tok_s = self.N / (self.flops / rate)
        return {"value": round(tok_s, 2), "unit": "tokens/s", **_oracle_threads(), "kind": "oracle",
                "sample": f"{rows_done} query rows x {self.HQ} heads of the {self.N}-token prompt (every {every}th "
                          f"query of its last two chunks, {flops:.3e} of its {self.flops:.3e} algorithmic FLOP): "
                          f"gather through the table + float64 attention in {t_total:.2f} s; the prompt's "
                          f"tokens/s is that FLOP rate applied to the whole prompt",
                "oracle_gflops": round(rate / 1e9, 2)}

    def check_last_chunk(self):
        import numpy as np
        import oracle as O
        c0 = ((self.N - 1) // self.CHUNK) * self.CHUNK
        self.chunk(c0)
        self.torch.cuda.synchronize()
        out = self.out.cpu().numpy()
        rows = np.array([0, 1, min(self.CHUNK, self.N - c0) - 1])
        w = self.w
        qc = np.ascontiguousarray(w.q[c0:c0 + self.CHUNK])
        qf = (qc.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = O.prefill(qf, w.as_f64("K")[0], w.as_f64("V")[0], c0, 1 / 16, rows=rows)
        return float(max(np.max(np.abs(out[r] - ref[r])) / np.max(np.abs(ref[r])) for r in rows))


# ---------------------------------------------------------------------------
# Block-sparse decode: pooling, scores + top-k, sparse attention
# ---------------------------------------------------------------------------

class SparseBench:
    """3 streams x 131072 cached positions, pages of 256 shuffled; indexer keys (128 wide) pooled per
    block of 4; 4 indexer heads score the pooled blocks; top-512 blocks; attention over their 2048 rows
    with 32 q / 4 KV heads, head dim 256, bf16."""
    S, L, PTOK, HQ, HKV, D, DI, HI, K = 3, 131072, 256, 32, 4, 256, 128, 4, 512

    def __init__(self, seed: int = 5):
        import numpy as np
        import torch
        import paged_kv_cache_pg_amd as P
        from paged_kv_cache_pg_amd.inputs import make_workload
        self.P, self.torch = P, torch
        t0 = time.time()
        w = make_workload(seed, [self.L] * self.S, self.PTOK, self.HQ, self.HKV, dtype="bf16", table_kind="shuffled",
                          idx_dim=self.DI, n_idx_heads=self.HI)
        self.w = w
        log(f"sparse: workload drawn in {time.time() - t0:.1f}s")
        lay = P.ArenaLayout(self.HKV, self.D, self.PTOK, P.PAGED_BF16, idx_dim=self.DI)
        self.table = torch.from_numpy(w.table.astype(np.int32)).cuda()
        self.pg = P.make_pg(self.table, self.PTOK, lay.page_elems)
        self.lens = torch.tensor(w.lens, dtype=torch.int32, device="cuda")
        zero = torch.zeros(self.S, dtype=torch.int32, device="cuda")
        self.arena = torch.zeros(w.n_pages * lay.page_bytes, dtype=torch.uint8, device="cuda")
        base = self.arena.data_ptr()
        for name, off, heads, width in (("K", lay.k_off, self.HKV, self.D), ("V", lay.v_off, self.HKV, self.D),
                                        ("IK", lay.ik_off, 1, self.DI)):
            src = torch.from_numpy(getattr(w, name).view(np.int16)).cuda()
            ss = heads * self.L * width
            P.paged_rows_store(src, ss, self.L * width if heads > 1 else 0, width, base + off, heads, width,
                               P.PAGED_BF16, self.pg, zero, self.lens, self.S, self.L)
            torch.cuda.synchronize()
            del src
        self.ik, self.pooled = base + lay.ik_off, base + lay.pool_off
        self.kv = P.make_kv(base + lay.k_off, base + lay.v_off, P.PAGED_BF16, self.HKV, self.D)
        self.q = torch.from_numpy(w.q.view(np.int16)).cuda()
        self.qi = torch.from_numpy(w.qI.view(np.int16)).cuda()
        self.b0 = zero
        self.b1 = torch.full((self.S,), self.L // 4, dtype=torch.int32, device="cuda")
        self.ids = torch.empty((self.S, self.K), dtype=torch.int32, device="cuda")
        self.cnt = torch.empty(self.S, dtype=torch.int32, device="cuda")
        self.scores = torch.empty((self.S, self.L // 4), dtype=torch.float64, device="cuda")
        self.tws = torch.empty(P.paged_topk_workspace(self.S, self.L, self.K), dtype=torch.uint8, device="cuda")
        self.sws = torch.empty(P.paged_sparse_attn_workspace(self.S, self.HQ, self.K), dtype=torch.uint8,
                               device="cuda")
        self.out = torch.empty((self.S, self.HQ, self.D), dtype=torch.float32, device="cuda")
        nb = self.S * (self.L // 4)
        self.bytes_pool = self.S * self.L * self.DI * 2 + nb * self.DI * 4
        self.bytes_scores = nb * self.DI * 4 + self.qi.numel() * 2 + nb * 8 + self.S * self.K * 4
        self.bytes_sparse = self.S * self.HKV * 4 * self.K * self.D * 2 * 2 + self.q.numel() * 2 + self.out.numel() * 4

    def pool(self, i=0):
        self.P.paged_pool_blocks(self.ik, self.pooled, self.DI, self.P.PAGED_BF16, self.pg, self.b0, self.b1, self.S,
                                 self.L)

    def scores_topk(self, i=0):
        self.P.paged_block_scores_topk(self.qi, self.P.PAGED_BF16, self.HI, self.DI, self.pooled, self.P.PAGED_BF16,
                                       self.pg, self.lens, self.S, self.L, self.K, self.ids, self.cnt, self.scores,
                                       self.tws)

    def sparse(self, i=0):
        self.P.paged_sparse_attn(self.q, self.P.PAGED_BF16, self.HQ, self.kv, self.pg, self.ids, self.cnt, self.K,
                                 self.S, self.L, 1 / 16, self.out, self.sws)

    def oracle_rate(self):
        """The oracle over the whole block-sparse step of all three streams: indexer keys gathered
        through the table and pooled, blocks scored, top-k selected, the selected K/V rows gathered
        and attended, all in float64."""
        import numpy as np
        import oracle as O
        from paged_kv_cache_pg_amd.inputs import bf16_bits_to_f32
        w = self.w
        olay = O.PageLayout(self.HKV, self.D, self.PTOK, "bf16", idx_dim=self.DI)
        arena = O.place(olay, w.table, w.n_pages, w.lens, w.K, w.V, w.IK)
        qf, qI = w.as_f64("q"), w.as_f64("qI")
        t0 = time.perf_counter()
        K, V, IK = O.gather(olay, w.table, arena, w.lens)
        pooled = O.pool(bf16_bits_to_f32(IK).astype(np.float64), w.lens)
        sel = [O.topk(O.scores(qI[s], pooled[s]), self.K) for s in range(self.S)]
        Ks = np.zeros((self.S, self.HKV, 4 * self.K, self.D))
        Vs = np.zeros_like(Ks)
        for s in range(self.S):
            pos = (4 * sel[s][:, None] + np.arange(4)[None, :]).reshape(-1)
            Ks[s] = bf16_bits_to_f32(K[s][:, pos]).astype(np.float64)
            Vs[s] = bf16_bits_to_f32(V[s][:, pos]).astype(np.float64)
        O.decode(qf, Ks, Vs, [4 * self.K] * self.S, 1 / 16)
        dt = time.perf_counter() - t0
        nbytes = self.bytes_pool + self.bytes_scores + self.bytes_sparse
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "us": round(dt * 1e6, 1), **_oracle_threads(),
                "kind": "oracle",
                "sample": f"one whole block-sparse step of the 3 x 131072 workload (pooling, scores, top-{self.K}, "
                          f"sparse attention; gathers through the table included) in {dt:.2f} s; GB/s of the "
                          f"step's algorithmic bytes ({nbytes})"}

    def check(self):
        """Top-k ids of stream 0 against the oracle (bit for bit), one sparse row within 2e-3."""
        import numpy as np
        import oracle as O
        self.pool(); self.scores_topk(); self.sparse()
        self.torch.cuda.synchronize()
        w = self.w
        pooled = O.pool(w.as_f64("IK")[:1], w.lens[:1])[0]
        want = O.topk(O.scores(w.as_f64("qI")[0], pooled), self.K)
        ids = self.ids.cpu().numpy()[0]
        ok = bool(np.array_equal(ids, want))
        pos = np.array([4 * b + j for b in want for j in range(4)])
        Ks = (w.K[0:1][:, :, pos].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        Vs = (w.V[0:1][:, :, pos].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = O.decode(w.as_f64("q")[0:1], Ks, Vs, [len(pos)], 1 / 16)[0]
        out = self.out.cpu().numpy()[0]
        err = float(np.max(np.max(np.abs(out - ref), axis=1) / np.max(np.abs(ref), axis=1)))
        return ok, err


class DecodeFp8Bench:
    """The decode workload with e4m3 rows (a float32 scale a row): 4 streams x 40960 positions, pages of 256
    shuffled in one arena, 32 q / 4 KV heads, head dim 256, bf16 q.  The rows are N(0,1) bf16 drawn on the
    device from a seeded generator and written by the library's own e4m3 store (paged_kv_append), through
    the table, so the arena holds what a serving loop would have stored."""
    S, L, PTOK, HQ, HKV, D = 4, 40960, 256, 32, 4, 256
    CHUNK = 4096

    def __init__(self, seed: int = 7):
        import numpy as np
        import torch
        import paged_kv_cache_pg_amd as P
        from paged_kv_cache_pg_amd.inputs import make_table
        self.P, self.torch, self.np = P, torch, np
        S, L = self.S, self.L
        rng = np.random.default_rng(seed)
        gen = torch.Generator(device="cuda").manual_seed(seed)
        self.table_np, n_pages = make_table("shuffled", [L // self.PTOK] * S, rng)
        self.lay = P.ArenaLayout(self.HKV, self.D, self.PTOK, P.PAGED_FP8_E4M3)
        self.table = torch.from_numpy(self.table_np.astype(np.int32)).cuda()
        self.pg = P.make_pg(self.table, self.PTOK, self.lay.page_elems)
        self.q = torch.randn((S, self.HQ, self.D), generator=gen, device="cuda").to(torch.bfloat16)
        self.lens = torch.full((S,), L, dtype=torch.int32, device="cuda")
        self.arenas, self.kvs = [], []
        for copy in range(2):
            arena = torch.zeros(n_pages * self.lay.page_bytes, dtype=torch.uint8, device="cuda")
            b = arena.data_ptr()
            kv = P.make_kv(b + self.lay.k_off, b + self.lay.v_off, P.PAGED_FP8_E4M3, self.HKV, self.D,
                           b + self.lay.ks_off, b + self.lay.vs_off)
            for p0 in range(0, L, self.CHUNK):
                shape = (S, self.CHUNK, self.HKV, self.D)
                k_new = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
                v_new = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
                pos0 = torch.full((S,), p0, dtype=torch.int32, device="cuda")
                P.paged_kv_append(k_new, v_new, None, self.CHUNK, kv, None, None, 0, self.pg, pos0, S, L)
                torch.cuda.synchronize()
            self.arenas.append(arena)
            self.kvs.append(kv)
        self.ws = torch.zeros(P.paged_attn_decode_workspace(S, self.HQ, L), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((S, self.HQ, self.D), dtype=torch.float32, device="cuda")
        self.alg_bytes = (S * self.HKV * L * (self.D + 4) * 2          # K and V codes and scales
                          + self.q.numel() * 2 + S * self.table_np.shape[1] * 4 + S * 4 + self.out.numel() * 4)

    def step(self, i: int):
        self.P.paged_attn_decode(self.q, self.P.PAGED_BF16, self.HQ, self.kvs[i & 1], self.pg, self.lens, self.S,
                                 self.L, 1 / 16, self.out, self.ws)

    def rows_of(self, arena, s: int, g: int):
        """The stored codes and scales of stream s, KV head g, read back through the table (host)."""
        import oracle as O
        np = self.np
        lay = O.PageLayout(self.HKV, self.D, self.PTOK, "fp8")
        kc = np.empty((self.L, self.D), np.uint8)
        vc = np.empty_like(kc)
        ks = np.empty(self.L, np.float32)
        vs = np.empty_like(ks)
        for lp in range(self.L // self.PTOK):
            p0 = lp * self.PTOK
            o = O.row_offset(self.table_np, self.PTOK, lay.page_elems, s, g, p0, self.D)
            so = O.row_offset(self.table_np, self.PTOK, lay.page_elems, s, g, p0, 4)
            kc[p0:p0 + self.PTOK] = arena[lay.k_off + o:lay.k_off + o + self.PTOK * self.D].reshape(self.PTOK, -1)
            vc[p0:p0 + self.PTOK] = arena[lay.v_off + o:lay.v_off + o + self.PTOK * self.D].reshape(self.PTOK, -1)
            ks[p0:p0 + self.PTOK] = arena[lay.ks_off + so:lay.ks_off + so + self.PTOK * 4].view(np.float32)
            vs[p0:p0 + self.PTOK] = arena[lay.vs_off + so:lay.vs_off + so + self.PTOK * 4].view(np.float32)
        return kc, vc, ks, vs

    def check(self):
        """Sampled rows against the oracle over the stored codes x scales (outside the timed region)."""
        import oracle as O
        np, torch = self.np, self.torch
        self.step(0)
        torch.cuda.synchronize()
        out = self.out.cpu().numpy()
        arena = self.arenas[0].cpu().numpy()
        q = self.q.float().cpu().numpy().astype(np.float64)
        worst = 0.0
        for s, h in [(0, 0), (3, 31)]:
            kc, vc, ks, vs = self.rows_of(arena, s, h // (self.HQ // self.HKV))
            ref = O.decode(q[s:s + 1, h:h + 1], O.e4m3_dequantize(kc, ks)[None, None],
                           O.e4m3_dequantize(vc, vs)[None, None], [self.L], 1 / 16)[0, 0]
            worst = max(worst, float(np.max(np.abs(out[s, h] - ref)) / np.max(np.abs(ref))))
        return worst


def run_sparse_fp8(dec, args, k: int = 512):
    """Sparse attention over the e4m3 decode workload: k blocks of 4 rows a stream (ascending ids drawn
    from a seeded generator), codes and scales read through the table; sampled rows against the oracle."""
    import numpy as np
    import torch
    P = dec.P
    rng = np.random.default_rng(11)
    ids = np.stack([np.sort(rng.choice(dec.L // 4, k, replace=False)) for _ in range(dec.S)]).astype(np.int32)
    ids_d = torch.from_numpy(ids).cuda()
    cnt = torch.full((dec.S,), k, dtype=torch.int32, device="cuda")
    ws = torch.zeros(P.paged_sparse_attn_workspace(dec.S, dec.HQ, k), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dec.out)

    def step(i):
        P.paged_sparse_attn(dec.q, P.PAGED_BF16, dec.HQ, dec.kvs[i & 1], dec.pg, ids_d, cnt, k, dec.S, dec.L, 1 / 16,
                            out, ws)
    ms, _ = time_steps(step, args.steps, args.warmup)
    nbytes = (dec.S * dec.HKV * 4 * k * (dec.D + 4) * 2 + dec.q.numel() * 2 + ids.size * 4 + dec.S * 4
              + out.numel() * 4)
    worst = None
    if ORACLE_LEG:
        import oracle as O
        step(0)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        arena = dec.arenas[0].cpu().numpy()
        q = dec.q.float().cpu().numpy().astype(np.float64)
        worst = 0.0
        for s, h in [(1, 5), (2, 30)]:
            kc, vc, ks, vs = dec.rows_of(arena, s, h // (dec.HQ // dec.HKV))
            pos = (4 * ids[s][:, None] + np.arange(4)[None, :]).reshape(-1)
            ref = O.decode(q[s:s + 1, h:h + 1], O.e4m3_dequantize(kc[pos], ks[pos])[None, None],
                           O.e4m3_dequantize(vc[pos], vs[pos])[None, None], [len(pos)], 1 / 16)[0, 0]
            worst = max(worst, float(np.max(np.abs(got[s, h] - ref)) / np.max(np.abs(ref))))
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"sparse e4m3 (k = {k}): {ms * 1e3:.1f} us, {gbs:.0f} GB/s; sampled rows within {_err(worst)} of the oracle")
    return {"k": k, "us": round(ms * 1e3, 2), "alg_bytes": nbytes, "GB_per_s": round(gbs, 1), "oracle_max_rel_err": worst}


class AppendBench:
    """paged_kv_append into pages of 256 (shuffled), 4 KV heads, head dim 256, 128-wide indexer keys, bf16:
    a decode step (4 streams x 1 token at position 4095, which completes a block of four) and a prefill chunk
    (1 stream x 2048 tokens at position 2048).  With fp8, the same steps into an e4m3 arena (bf16 rows in,
    codes and a float32 scale a row out, no indexer keys)."""
    HKV, D, DI, PTOK = 4, 256, 128, 256

    def __init__(self, n_streams: int, n_new: int, pos0: int, seed: int = 6, fp8: bool = False):
        import numpy as np
        import torch
        import paged_kv_cache_pg_amd as P
        from paged_kv_cache_pg_amd.inputs import make_table
        self.P, self.torch = P, torch
        S, L = n_streams, pos0 + n_new
        self.fp8 = fp8
        if fp8:
            lay = P.ArenaLayout(self.HKV, self.D, self.PTOK, P.PAGED_FP8_E4M3)
        else:
            lay = P.ArenaLayout(self.HKV, self.D, self.PTOK, P.PAGED_BF16, idx_dim=self.DI)
        rng = np.random.default_rng(seed)
        table, n_pages = make_table("shuffled", [(L + self.PTOK - 1) // self.PTOK] * S, rng)
        self.table = torch.from_numpy(table.astype(np.int32)).cuda()
        self.pg = P.make_pg(self.table, self.PTOK, lay.page_elems)
        self.arena = torch.zeros(n_pages * lay.page_bytes, dtype=torch.uint8, device="cuda")
        base = self.arena.data_ptr()
        self.k_new = torch.randn((S, n_new, self.HKV, self.D), device="cuda").to(torch.bfloat16)
        self.v_new = torch.randn((S, n_new, self.HKV, self.D), device="cuda").to(torch.bfloat16)
        self.pos0 = torch.full((S,), pos0, dtype=torch.int32, device="cuda")
        self.S, self.n, self.L = S, n_new, L
        if fp8:
            self.kv = P.make_kv(base + lay.k_off, base + lay.v_off, P.PAGED_FP8_E4M3, self.HKV, self.D,
                                base + lay.ks_off, base + lay.vs_off)
            self.ik = self.pooled = self.ik_new = None
            # bf16 K and V rows read once, codes and scales written once
            self.bytes = S * n_new * 2 * self.HKV * (self.D * 2 + self.D + 4)
            return
        self.kv = P.make_kv(base + lay.k_off, base + lay.v_off, P.PAGED_BF16, self.HKV, self.D)
        self.ik, self.pooled = base + lay.ik_off, base + lay.pool_off
        self.ik_new = torch.randn((S, n_new, self.DI), device="cuda").to(torch.bfloat16)
        n_blocks = S * ((pos0 + n_new) // 4 - pos0 // 4)
        # K, V and indexer-key rows read and written once, pooled rows written once
        self.bytes = 2 * S * n_new * (2 * self.HKV * self.D * 2 + self.DI * 2) + n_blocks * self.DI * 4

    def step(self, i=0):
        self.P.paged_kv_append(self.k_new, self.v_new, self.ik_new, self.n, self.kv, self.ik, self.pooled, self.DI,
                               self.pg, self.pos0, self.S, self.L)


def time_graph(fn, steps: int, warmup: int):
    """K calls captured in one HIP graph and replayed, timed with HIP events around a replay: the GPU
    time of calls too short for the host to issue back to back (the calls allocate nothing and record
    no memset)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(1, warmup)):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def run_append(args):
    out = {}
    for name, (S, n, p0, fp8) in (("decode_step_4x1", (4, 1, 4095, False)),
                                  ("prefill_chunk_1x2048", (1, 2048, 2048, False)),
                                  ("decode_step_4x1_e4m3", (4, 1, 4095, True)),
                                  ("prefill_chunk_1x2048_e4m3", (1, 2048, 2048, True))):
        ab = AppendBench(S, n, p0, fp8=fp8)
        ms = time_graph(ab.step, args.steps, args.warmup)
        out[name] = {"us": round(ms * 1e3, 2), "bytes": ab.bytes, "GB_per_s": round(ab.bytes / (ms * 1e-3) / 1e9, 1)}
        log(f"append {name}: {ms * 1e3:.1f} us, {ab.bytes / (ms * 1e-3) / 1e9:.0f} GB/s")
        del ab
    return out


def time_steps(fn, steps: int, warmup: int):
    """Warm-up, then K steps bracketed by a synchronize and a pair of HIP events on the current stream
    (the stream the library launches on).  Returns (ms per step, wall seconds)."""
    import torch
    # at least `warmup` steps and at least 0.3 s of them, so clocks have settled after host-side work
    t_w = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_w < 0.3:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, time.perf_counter() - t0


def time_launches(fn, n: int):
    """Per-launch HIP event pairs around each call (the events' own packets fall between launches)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    return sum(per) / n, per[0], per[n // 2]


def run_window(dec, args, W: int = 2):
    """The decode workload with a window of W queries a stream (drafted tokens verified at once): K/V
    are read once for all W queries."""
    import torch
    P = dec.P
    q = torch.randn((dec.S, W, dec.HQ, dec.D), device="cuda").to(torch.bfloat16)
    ws = torch.zeros(P.paged_attn_decode_window_workspace(dec.S, dec.HQ, W, dec.L), dtype=torch.uint8, device="cuda")
    out = torch.empty((dec.S, W, dec.HQ, dec.D), dtype=torch.float32, device="cuda")

    def step(i):
        P.paged_attn_decode_window(q, P.PAGED_BF16, dec.HQ, W, dec.kvs[i & 1], dec.pg, dec.lens, dec.S, dec.L, 1 / 16,
                                   out, ws)
    ms, _ = time_steps(step, args.steps, args.warmup)
    nbytes = dec.alg_bytes + dec.q.numel() * 2 * (W - 1) + dec.out.numel() * 4 * (W - 1)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"decode window {W}: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s, {dec.S * W / (ms * 1e-3):.0f} tokens/s")
    return {"window": W, "us_per_step": round(ms * 1e3, 2), "alg_bytes": nbytes, "GB_per_s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "tokens_per_s": round(dec.S * W / (ms * 1e-3), 1)}


def run_rows(dec, args):
    """Page-run save and restore of the decode workload's cache: every K and V row of the 4 streams
    gathered from the paged arena into the contiguous layout [S][Hkv][L][D], then stored through the
    table into a zeroed arena, which must come out equal to the first byte for byte."""
    import torch
    P = dec.P
    S, H, L, D = dec.S, dec.HKV, dec.L, dec.D
    lay = dec.lay
    cont = torch.empty((2, S, H, L, D), dtype=torch.int16, device="cuda")
    begin = torch.zeros(S, dtype=torch.int32, device="cuda")
    src = dec.arenas[0]
    dst = torch.zeros_like(src)
    regions = ((0, lay.k_off), (1, lay.v_off))

    def save(i):
        for j, off in regions:
            P.paged_rows_gather(cont[j], H * L * D, L * D, D, src.data_ptr() + off, H, D, P.PAGED_BF16, dec.pg,
                                begin, dec.lens, S, L)

    def restore(i):
        for j, off in regions:
            P.paged_rows_store(cont[j], H * L * D, L * D, D, dst.data_ptr() + off, H, D, P.PAGED_BF16, dec.pg,
                               begin, dec.lens, S, L)
    out = {}
    moved = 2 * cont.numel() * 2  # bytes read + bytes written
    for name, fn in (("save_gather", save), ("restore_store", restore)):
        ms, _ = time_steps(fn, max(1, args.steps // 4), max(1, args.warmup // 4))
        out[name] = {"us": round(ms * 1e3, 1), "bytes_moved": moved, "GB_per_s": round(moved / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"rows {name}: {ms * 1e3:.1f} us, {moved / (ms * 1e-3) / 1e9:.0f} GB/s")
    torch.cuda.synchronize()
    out["restored_equals_original"] = bool(torch.equal(dst, src))
    del cont, dst
    torch.cuda.empty_cache()
    return out


def _sclk_now():
    """Current shader clock levels (MHz) of the GPUs sysfs lists (the level marked '*'), or []."""
    import glob
    import re
    out = []
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(f) as fh:
                for line in fh:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*mhz", line, re.I)
                        if m:
                            out.append(int(m.group(1)))
        except OSError:
            pass
    return out


class ClockSampler:
    """Samples the highest current shader clock sysfs reports every 20 ms on a background thread."""

    def __init__(self, what: str = "decode steps"):
        import threading
        self.what = what
        self.samples, self._stop = [], threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.wait(0.02):
            c = _sclk_now()
            if c:
                self.samples.append(max(c))

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        import statistics
        if not self.samples:
            return None
        return {"median": statistics.median(self.samples), "min": min(self.samples), "max": max(self.samples),
                "samples": len(self.samples),
                "source": f"sysfs pp_dpm_sclk current level, every 20 ms during the timed {self.what}"}


def run_page_pool():
    """The host page pool (no GPU): a pool of 65,536 pages; alloc then free of n pages in one call each,
    and claim then release of a run of k pages, repeated; pages (or runs) handled per second and the
    time per call pair, ctypes calls included."""
    import numpy as np
    import paged_kv_cache_pg_amd as P
    n_pages = 65536
    state = np.zeros(P.paged_pool_state_bytes(n_pages), np.uint8)
    P.paged_pool_init(state, n_pages)
    out = {}
    for n in (1, 64, 1024):
        pages = np.zeros(n, np.int32)
        reps = max(200, 200000 // n)
        t0 = time.perf_counter()
        for _ in range(reps):
            P.paged_pool_alloc(state, n, pages)
            P.paged_pool_free(state, pages, n)
        dt = time.perf_counter() - t0
        out[f"alloc_free_{n}"] = {"us_per_pair": round(dt / reps * 1e6, 3), "pages_per_s": round(reps * n / dt, 1)}
    for k in (4, 64):
        reps = 20000
        t0 = time.perf_counter()
        for _ in range(reps):
            first = P.paged_pool_claim_run(state, k)
            P.paged_pool_release_run(state, first, k)
        dt = time.perf_counter() - t0
        out[f"claim_release_run_{k}"] = {"us_per_pair": round(dt / reps * 1e6, 3)}
    assert P.paged_pool_free_count(state) == n_pages
    log(f"page pool: alloc+free of 1024 pages {out['alloc_free_1024']['us_per_pair']} us, "
        f"claim+release of a 64-page run {out['claim_release_run_64']['us_per_pair']} us")
    return out


def run_decode(args):
    import torch
    dec = DecodeBench()
    with ClockSampler() as clk:
        ms_step, wall = time_steps(dec.step, args.steps, args.warmup)
    ms_call, ms_min, ms_med = time_launches(dec.step, max(args.steps, 20))
    err = dec.check() if ORACLE_LEG else None
    log(f"decode: sampled rows within {_err(err)} of the oracle")
    gbs = dec.alg_bytes / (ms_step * 1e-3) / 1e9
    call_gbs = dec.alg_bytes / (ms_call * 1e-3) / 1e9
    log(f"decode: {ms_step * 1e3:.1f} us/step, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM peak)")
    out = {
        "value": round(gbs, 2),
        "ms_per_step": round(ms_step, 5),
        "roofline": {"bound": "hbm", "achieved": round(call_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(call_gbs / HBM_PEAK_GBS, 4),
                     "traffic": DECODE_TRAFFIC_BYTES if _decode_sources_hash() == DECODE_TRAFFIC_SOURCES else None,
                     "kernel": "paged_attn_decode (split + combine)", "alg_bytes_per_launch": dec.alg_bytes,
                     "avg_launch_us": round(ms_call * 1e3, 2), "min_launch_us": round(ms_min * 1e3, 2),
                     "median_launch_us": round(ms_med * 1e3, 2)},
        "oracle_max_rel_err": err,
        "gpu_sclk_mhz": clk.summary(),
        "decode_window": run_window(dec, args),
        "page_runs": run_rows(dec, args),
    }
    del dec
    torch.cuda.empty_cache()
    out["decode_batch_shapes"] = run_decode_batches(args)
    return out


def run_decode_batches(args, streams=(1, 2, 3, 5, 8)):
    """The headline decode's shape (40960 positions a stream, pages of 256 shuffled, 32 q / 4 KV heads,
    bf16) at other batch sizes.  Every page of the arena holds N(0,1) bf16 rows drawn on the device;
    enough arena copies rotate between steps that the 256 MB Infinity Cache cannot serve a step from
    the previous one.  One (stream, head) row of each shape is checked against the oracle."""
    import numpy as np
    import torch
    import paged_kv_cache_pg_amd as P
    from paged_kv_cache_pg_amd.inputs import make_table
    L, PT, HQ, HKV, D = 40960, 256, 32, 4, 256
    lay = P.ArenaLayout(HKV, D, PT, P.PAGED_BF16)
    gen = torch.Generator(device="cuda").manual_seed(21)
    out = {}
    for S in streams:
        table_np, n_pages = make_table("shuffled", [L // PT] * S, np.random.default_rng(100 + S))
        table = torch.from_numpy(table_np.astype(np.int32)).cuda()
        pg = P.make_pg(table, PT, lay.page_elems)
        arena_bytes = n_pages * lay.page_bytes
        copies = max(2, -(-600_000_000 // arena_bytes))
        arenas = [torch.randn(arena_bytes // 2, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(copies)]
        kvs = [P.make_kv(a.data_ptr() + lay.k_off, a.data_ptr() + lay.v_off, P.PAGED_BF16, HKV, D) for a in arenas]
        q = torch.randn((S, HQ, D), generator=gen, device="cuda").to(torch.bfloat16)
        lens = torch.full((S,), L, dtype=torch.int32, device="cuda")
        ws = torch.zeros(P.paged_attn_decode_workspace(S, HQ, L), dtype=torch.uint8, device="cuda")
        o = torch.empty((S, HQ, D), dtype=torch.float32, device="cuda")

        def step(i):
            P.paged_attn_decode(q, P.PAGED_BF16, HQ, kvs[i % copies], pg, lens, S, L, 1 / 16, o, ws)
        ms, _ = time_steps(step, args.steps, args.warmup)
        nbytes = S * HKV * L * D * 2 * 2 + q.numel() * 2 + table.numel() * 4 + S * 4 + o.numel() * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        # one row against the oracle: the last stream's last head, its rows read back through the table
        err = None
        if ORACLE_LEG:
            import oracle as O
            step(0)
            torch.cuda.synchronize()
            s, h = S - 1, HQ - 1
            g = h // (HQ // HKV)
            a0 = arenas[0].view(torch.int16).cpu().numpy().view(np.uint16)
            pe = lay.page_elems
            Kr = np.concatenate([a0[int(table_np[s, lp]) * pe + (lay.k_off // 2) + g * PT * D:][:PT * D] for lp in range(L // PT)])
            Vr = np.concatenate([a0[int(table_np[s, lp]) * pe + (lay.v_off // 2) + g * PT * D:][:PT * D] for lp in range(L // PT)])
            f64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            qf = q[s:s + 1, h:h + 1].float().cpu().numpy().astype(np.float64)
            ref = O.decode(qf, f64(Kr).reshape(1, 1, L, D), f64(Vr).reshape(1, 1, L, D), [L], 1 / 16)[0, 0]
            got = o[s, h].cpu().numpy()
            err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
            del a0
        out[str(S)] = {"streams": S, "us_per_step": round(ms * 1e3, 2), "alg_bytes": nbytes, "GB_per_s": round(gbs, 1),
                       "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "arena_copies": copies, "oracle_row_rel_err": err}
        log(f"decode {S} x {L}: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%}); row err {_err(err)}")
        del arenas, kvs
        torch.cuda.empty_cache()
    return out


def run_decode_fp8(args):
    dec = DecodeFp8Bench()
    ms_step, _ = time_steps(dec.step, args.steps, args.warmup)
    ms_call, ms_min, ms_med = time_launches(dec.step, max(args.steps, 20))
    err = dec.check() if ORACLE_LEG else None
    gbs = dec.alg_bytes / (ms_step * 1e-3) / 1e9
    call_gbs = dec.alg_bytes / (ms_call * 1e-3) / 1e9
    log(f"decode e4m3: {ms_step * 1e3:.1f} us/step, {gbs:.0f} GB/s ({call_gbs / HBM_PEAK_GBS:.1%} of HBM peak a "
        f"launch); sampled rows within {_err(err)} of the oracle")
    out = {"us_per_step": round(ms_step * 1e3, 2), "GB_per_s": round(gbs, 1), "alg_bytes_per_launch": dec.alg_bytes,
           "avg_launch_us": round(ms_call * 1e3, 2), "median_launch_us": round(ms_med * 1e3, 2),
           "hbm_frac": round(call_gbs / HBM_PEAK_GBS, 4), "oracle_max_rel_err": err,
           "tokens_per_s": round(dec.S / (ms_step * 1e-3), 1),
           "traffic": FP8_TRAFFIC_BYTES if _sources_hash(_FP8_SOURCES) == FP8_TRAFFIC_SOURCES else None,
           "sparse_attn_e4m3": run_sparse_fp8(dec, args)}
    del dec
    return out


def time_runs(fn, runs: int, warmup: int = 1):
    """Each of `runs` calls bracketed by its own pair of HIP events on the current stream (the
    stream the library launches on); returns the per-run times in ms, sorted."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for i in range(runs):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in evs)


def run_prefill(args, cpu_baseline: bool = False):
    import statistics
    import torch
    prefill = {}
    runs = max(5, args.steps // 4)
    for n_tok in (8192, 40960):
        pb = PrefillBench(n_tok)
        with ClockSampler("prompt runs") as clk:
            per = time_runs(pb.run, runs)
        ms = statistics.median(per)
        perr = pb.check_last_chunk() if ORACLE_LEG else None
        tflops = pb.flops / (ms * 1e-3) / 1e12
        prefill[str(n_tok)] = {"tokens_per_s": round(n_tok / (ms * 1e-3), 1), "ms": round(ms, 3),
                               "ms_min": round(per[0], 3), "ms_max": round(per[-1], 3), "runs": runs,
                               "tokens_per_s_best": round(n_tok / (per[0] * 1e-3), 1),
                               "chunks": (n_tok + 2047) // 2048, "alg_tflops": round(tflops, 1),
                               "mfma_util": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "oracle_max_rel_err": perr,
                               "gpu_sclk_mhz": clk.summary()}
        log(f"prefill {n_tok}: median {ms:.2f} ms (min {per[0]:.2f}) over {runs} runs, {n_tok / (ms * 1e-3):.0f} "
            f"tok/s, {tflops:.0f} TFLOP/s ({tflops / MFMA_BF16_PEAK_TFLOPS:.1%} of bf16 MFMA peak)")
        if cpu_baseline and n_tok == 40960:
            prefill[str(n_tok)]["cpu_baseline"] = cb = pb.oracle_rate()
            log(f"prefill {n_tok}: oracle {cb['value']:.1f} tokens/s ({cb['oracle_gflops']} GFLOP/s)")
        del pb
        torch.cuda.empty_cache()
    return prefill


def run_sparse(args, cpu_baseline: bool = False):
    sb = SparseBench()
    sparse = {}
    total_us = 0.0
    for name, fn, nbytes in (("pool_blocks", sb.pool, sb.bytes_pool), ("scores_topk", sb.scores_topk, sb.bytes_scores),
                             ("sparse_attn", sb.sparse, sb.bytes_sparse)):
        ms, _ = time_steps(fn, args.steps, args.warmup)
        sparse[name] = {"us": round(ms * 1e3, 2), "alg_bytes": nbytes, "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        if name != "pool_blocks":
            total_us += ms * 1e3
        log(f"sparse {name}: {ms * 1e3:.1f} us, {nbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
    # dense decode of the same streams (every cached row), the bytes the selection avoids
    import torch
    P = sb.P
    dws = torch.zeros(P.paged_attn_decode_workspace(sb.S, sb.HQ, sb.L), dtype=torch.uint8, device="cuda")
    dout = torch.empty_like(sb.out)

    def dense(i):
        P.paged_attn_decode(sb.q, P.PAGED_BF16, sb.HQ, sb.kv, sb.pg, sb.lens, sb.S, sb.L, 1 / 16, dout, dws)
    ms, _ = time_steps(dense, args.steps, args.warmup)
    dbytes = sb.S * sb.HKV * sb.L * sb.D * 2 * 2 + sb.q.numel() * 2 + sb.S * (sb.L // sb.PTOK) * 4 + sb.S * 4 + dout.numel() * 4
    sparse["dense_decode_131072"] = {"us": round(ms * 1e3, 2), "alg_bytes": dbytes,
                                     "GB_per_s": round(dbytes / (ms * 1e-3) / 1e9, 1),
                                     "hbm_frac": round(dbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"dense decode over the same 3 x 131072 streams: {ms * 1e3:.1f} us, {dbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
    del dws, dout
    ids_ok, serr = sb.check() if ORACLE_LEG else (None, None)
    sparse["decode_total_us"] = round(total_us, 2)
    sparse["topk_ids_equal_oracle"] = ids_ok
    sparse["oracle_max_rel_err"] = serr
    log(f"sparse: scores + top-k + attention {total_us:.1f} us; ids == oracle: {ids_ok}; err {_err(serr)}")
    if cpu_baseline:
        sparse["cpu_baseline"] = cb = sb.oracle_rate()
        log(f"sparse: oracle {cb['us'] / 1e6:.2f} s a step, {cb['value']} GB/s")
    del sb
    return sparse


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode", "decode_batches", "decode_fp8", "prefill", "sparse", "append"],
                    default=None,
                    help="run one row only (for profiler runs)")
    args = ap.parse_args()
    global ORACLE_LEG
    ORACLE_LEG = not args.no_cpu_baseline
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    result = {
        "metric": "paged decode KV GB/s (% of HBM peak) and prefill tokens/s at 40960 ctx",
        "value": None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "batched paged decode: 4 streams x 40960 cached positions, pages of 256 shuffled in "
                               "one arena, 32 q / 4 KV heads, head dim 256, bf16 K/V/q, fp32 accumulation",
                   "streams": 4, "seq_len": 40960, "page_pos": 256, "q_heads": 32, "kv_heads": 4, "head_dim": 256,
                   "parallelism": "single GPU"},
    }
    if args.only in (None, "decode"):
        result.update(run_decode(args))
        torch.cuda.empty_cache()
    if args.only == "decode_batches":
        result["decode_batch_shapes"] = run_decode_batches(args)
    if args.only in (None, "decode_fp8"):
        result["decode_e4m3"] = run_decode_fp8(args)
        torch.cuda.empty_cache()
    want_cpu = args.only is None and not args.no_cpu_baseline
    if args.only in (None, "prefill"):
        result["prefill"] = run_prefill(args, cpu_baseline=want_cpu)
        torch.cuda.empty_cache()
    if args.only in (None, "sparse"):
        result["sparse"] = run_sparse(args, cpu_baseline=want_cpu)
        torch.cuda.empty_cache()
    if args.only in (None, "append"):
        result["append"] = run_append(args)
        result["page_pool"] = run_page_pool()
        torch.cuda.empty_cache()
    if want_cpu:
        result["cpu_baseline"] = DecodeBench.cpu_baseline_from_scratch()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
