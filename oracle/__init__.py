"""float64 CPU oracle for paged KV-cache attention -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg (the oracle timed on the host and
the spot checks of sampled rows, both off with --no-cpu-baseline) may import this package.
"""
from .paged_oracle import (  # noqa: F401
    ESIZE,
    PageLayout,
    row_offset,
    pool_row_offset,
    place,
    gather,
    read_pooled,
    decode,
    decode_window,
    prefill,
    sparse,
    pool,
    scores,
    topk,
    E4M3_MAX,
    e4m3_value,
    e4m3_encode,
    e4m3_quantize_rows,
    e4m3_dequantize,
    place_fp8,
    gather_fp8,
)
