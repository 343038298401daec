"""The oracle's pins catch plausible mistakes: each case plants one mistake in an oracle function
(on the CPU, through a wrapper that swaps the module attribute the pins call) and requires that at
least one of the pins written for that function then fails.  The unmodified oracle passes the same
pins in tests/test_oracle_pins.py and tests/test_oracle_fp8.py."""
import numpy as np
import pytest

import oracle as O
import test_oracle_fp8 as F
import test_oracle_pins as T

_decode, _window, _prefill, _sparse = O.decode, O.decode_window, O.prefill, O.sparse
_pool, _scores, _topk = O.pool, O.scores, O.topk
_row_offset, _e4m3_value, _e4m3_encode = O.row_offset, O.e4m3_value, O.e4m3_encode
_pool_row_offset, _place, _gather, _quantize = O.pool_row_offset, O.place, O.gather, O.e4m3_quantize_rows
_dequantize = O.e4m3_dequantize


def _gather_swapped(*a, **k):
    K, V, IK = _gather(*a, **k)
    return V, K, IK


def _quantize_447(x):
    """Row scale amax / 447 instead of amax / 448."""
    codes, scales = _quantize(x)
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, (amax / np.float32(447)).astype(np.float32), np.float32(0))
    div = np.where(amax > 0, scale, np.float32(1))[..., None]
    return np.asarray(_e4m3_encode((x / div).astype(np.float32))).astype(np.uint8), scale.astype(np.float32)


def _window_one_back(q, K, V, lens, scale):
    """Window query w stands one position early (sees keys 0 .. L - W + w - 1)."""
    return _window(q, K, V, [max(int(l) - 1, 0) for l in lens], scale)


def _head_modulo(q, K, V, lens, scale):
    """Query head h reads KV head h mod Hkv instead of h // G."""
    Hq, Hkv = q.shape[1], K.shape[1]
    idx = [h % Hkv for h in range(Hq)]
    return _decode(q, K[:, idx], V[:, idx], lens, scale)


def _scores_one_accumulator(qI, pooled):
    """One float64 accumulator per block, head by head and dim by dim."""
    P = pooled.astype(np.float64)
    acc = np.zeros(P.shape[0])
    for h in range(qI.shape[0]):
        for d in range(qI.shape[1]):
            acc = acc + qI[h, d] * P[:, d]
    return acc


def _scores_groups_in_sequence(qI, pooled):
    """The stated heads-first sum and 8 chunk groups, but the groups added one after the other."""
    P = pooled.astype(np.float64)
    q = np.zeros(qI.shape[1])
    for h in range(qI.shape[0]):
        q = q + qI[h]
    prod = P * q[None, :]
    total = np.zeros(P.shape[0])
    for j in range(8):
        acc = np.zeros(P.shape[0])
        for c in range(j, (qI.shape[1] + 3) // 4, 8):
            for d in range(4 * c, min(4 * c + 4, qI.shape[1])):
                acc = acc + prod[:, d]
        total = total + acc
    return total


def _topk_ties_high(score, k):
    order = sorted(range(len(score)), key=lambda b: (-score[b], -b))
    return np.sort(np.array(order[:min(k, len(score))], dtype=np.int64))


def _topk_score_order(score, k):
    order = sorted(range(len(score)), key=lambda b: (-score[b], b))
    return np.array(order[:min(k, len(score))], dtype=np.int64)


def _prefill_causal_one_late(q, K, V, q_pos0, scale, causal=True, rows=None):
    """The query at position p also sees key p + 1 (where it is stored)."""
    if not causal:
        return _prefill(q, K, V, q_pos0, scale, causal, rows)
    Nq, Hq, D = q.shape
    G = Hq // K.shape[0]
    Lk = q_pos0 + Nq
    out = np.zeros((Nq, Hq, D))
    sel = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    for h in range(Hq):
        g = h // G
        z = scale * (q[sel, h] @ K[g, :Lk].T)
        z = np.where(np.arange(Lk)[None, :] > (q_pos0 + sel)[:, None] + 1, -np.inf, z)
        e = np.exp(z - z.max(axis=1, keepdims=True))
        out[sel, h] = (e @ V[g, :Lk]) / e.sum(axis=1, keepdims=True)
    return out


def _prefill_head_modulo(q, K, V, q_pos0, scale, causal=True, rows=None):
    """Query head h reads KV head h mod Hkv instead of h // G."""
    idx = [h % K.shape[0] for h in range(q.shape[1])]
    return _prefill(q, K[idx], V[idx], q_pos0, scale, causal, rows)


def _topk_one_short(score, k):
    ids = _topk(score, k)
    return ids[:-1] if len(ids) else ids


def _e4m3_no_saturation(y):
    y = np.asarray(y, dtype=np.float64)
    c = np.asarray(_e4m3_encode(y)).copy()
    big = np.abs(y) > 448
    c[big] = np.where(y[big] < 0, 0xFF, 0x7F)   # NaN codes instead of +-448
    return c


def _window_attends_whole_cache(q, K, V, lens, scale):
    S, W = q.shape[:2]
    return np.stack([_decode(q[:, w], K, V, lens, scale) for w in range(W)], axis=1)


BRUTE = [lambda: T.test_decode_matches_50_digit_brute_force(4, 5, 2),
         lambda: T.test_decode_matches_50_digit_brute_force(8, 12, 4)]
DECODE_PINS = [T.test_decode_single_key_is_value_row, T.test_decode_zero_query_is_mean_of_values_over_exactly_L_rows,
               T.test_decode_two_keys_logistic_closed_form, T.test_decode_gqa_head_map_is_division,
               T.test_decode_dominant_key_and_affine_equivariance, T.test_decode_empty_stream_is_zero, *BRUTE]

SCORES_PINS = [T.test_scores_exact_on_integers_and_linear_in_heads,
               T.test_scores_sum_order_heads_first_then_eight_groups_and_a_tree]

MUTANTS = {
    "decode drops the scale": ("decode", lambda q, K, V, lens, scale: _decode(q, K, V, lens, 1.0), DECODE_PINS),
    "decode doubles the scale": ("decode", lambda q, K, V, lens, scale: _decode(q, K, V, lens, 2 * scale), DECODE_PINS),
    "decode reads one key too few": ("decode", lambda q, K, V, lens, scale:
                                     _decode(q, K, V, [max(int(l) - 1, 0) for l in lens], scale), DECODE_PINS),
    "decode maps heads modulo": ("decode", _head_modulo, DECODE_PINS),
    "decode swaps keys and values": ("decode", lambda q, K, V, lens, scale: _decode(q, V, K, lens, scale), DECODE_PINS),
    "prefill drops the causal mask": ("prefill", lambda q, K, V, q_pos0, scale, causal=True, rows=None:
                                      _prefill(q, K, V, q_pos0, scale, False, rows),
                                      [T.test_prefill_first_row_and_causal_mask_offsets,
                                       T.test_prefill_rows_equal_decode_and_chunking_invariance]),
    "window queries see the whole cache": ("decode_window", _window_attends_whole_cache,
                                           [T.test_decode_window_closed_form_and_short_streams,
                                            T.test_decode_window_equals_causal_prefill_and_decode,
                                            T.test_decode_window_matches_50_digit_brute_force]),
    "sparse ignores the block ids": ("sparse", lambda q, K, V, ids, scale:
                                     _decode(q, K, V, [K.shape[2]] * q.shape[0], scale),
                                     [T.test_sparse_all_blocks_is_dense_and_subset_is_row_restriction]),
    "pool divides by 3": ("pool", lambda IK, lens: [None if x is None else np.float32(x * (4 / 3))
                                                    for x in _pool(IK, lens)],
                          [T.test_pool_closed_forms, T.test_pool_of_short_stream_is_empty]),
    "scores sum the dims backwards": ("scores", lambda qI, pooled:
                                      _scores(np.ascontiguousarray(qI[:, ::-1]), np.ascontiguousarray(pooled[:, ::-1])),
                                      SCORES_PINS),
    "scores in one accumulator head by head": ("scores", _scores_one_accumulator, SCORES_PINS),
    "scores groups added in sequence": ("scores", _scores_groups_in_sequence, SCORES_PINS),
    "scores drop a head": ("scores", lambda qI, pooled: _scores(qI[:-1], pooled) if len(qI) > 1 else _scores(qI, pooled),
                           SCORES_PINS),
    "top-k ties go to the higher id": ("topk", _topk_ties_high, [T.test_topk_matches_python_sort_and_ties]),
    "top-k ids in score order": ("topk", _topk_score_order, [T.test_topk_matches_python_sort_and_ties]),
    "row offset one row off": ("row_offset", lambda *a, **k: _row_offset(*a, **k) + a[6],
                               [T.test_row_offset_hand_derived]),
    "e4m3 exponent bias 8": ("e4m3_value", lambda c: np.asarray(_e4m3_value(c)) * 0.5,
                             [F.test_e4m3_values_derived_by_hand, F.test_e4m3_values_match_torch_float8_e4m3fn]),
    "pooled-row offset one row off": ("pool_row_offset", lambda *a, **k: _pool_row_offset(*a, **k) + a[5],
                                      [T.test_pool_row_offset_hand_derived]),
    "place swaps keys and values": ("place", lambda lay, table, n, lens, K, V, IK=None:
                                    _place(lay, table, n, lens, V, K, IK),
                                    [lambda: T.test_place_gather_round_trip("shuffled", 12),
                                     lambda: T.test_place_gather_round_trip("reversed", 4)]),
    "gather swaps keys and values": ("gather", _gather_swapped,
                                     [lambda: T.test_place_gather_round_trip("shuffled", 12),
                                      lambda: T.test_place_gather_round_trip("identity", 16)]),
    "window queries one position early": ("decode_window", _window_one_back,
                                          [T.test_decode_window_closed_form_and_short_streams,
                                           T.test_decode_window_equals_causal_prefill_and_decode,
                                           T.test_decode_window_matches_50_digit_brute_force]),
    "e4m3 row scale amax / 447": ("e4m3_quantize_rows", _quantize_447,
                                  [F.test_quantize_rows_invariants, F.test_quantize_rows_special_rows]),
    "e4m3 encode does not saturate": ("e4m3_encode", _e4m3_no_saturation,
                                      [F.test_e4m3_encode_ties_go_to_the_even_code_and_large_values_saturate]),
    "prefill causal mask one key late": ("prefill", _prefill_causal_one_late,
                                         [T.test_prefill_first_row_and_causal_mask_offsets,
                                          T.test_prefill_rows_equal_decode_and_chunking_invariance]),
    "prefill maps heads modulo": ("prefill", _prefill_head_modulo,
                                  [T.test_prefill_first_row_and_causal_mask_offsets,
                                   T.test_prefill_rows_equal_decode_and_chunking_invariance]),
    "sparse rows one position late": ("sparse", lambda q, K, V, ids, scale:
                                      _sparse(q, np.roll(K, -1, axis=2), np.roll(V, -1, axis=2), ids, scale),
                                      [T.test_sparse_all_blocks_is_dense_and_subset_is_row_restriction]),
    "pool over rows one position late": ("pool", lambda IK, lens: _pool(np.roll(IK, -1, axis=1), lens),
                                         [T.test_pool_closed_forms, T.test_pool_of_short_stream_is_empty]),
    "top-k returns one id too few": ("topk", _topk_one_short, [T.test_topk_matches_python_sort_and_ties]),
    "e4m3 dequantize ignores the row scale": ("e4m3_dequantize", lambda codes, scales: _e4m3_value(codes) * 1.0,
                                              [F.test_quantize_rows_invariants]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_a_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, mutant, pins = MUTANTS[name]
    monkeypatch.setattr(O, attr, mutant)
    failed = []
    for pin in pins:
        try:
            pin()
        except AssertionError:  # only a pin's own check counts; any other error is a broken case
            failed.append(getattr(pin, "__name__", "pin"))
    assert failed, f"no pin caught: {name}"
