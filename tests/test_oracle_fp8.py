"""Pins of the oracle's e4m3 functions to things other than themselves: codes derived by hand from
the OCP E4M3 definition, torch's own float8_e4m3fn conversions (a library routine), an exhaustive
round trip, ties, saturation, and the quantizer's invariants (its largest code, its error bound)."""
import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_pg_amd.inputs import draw_e4m3_codes, draw_row_scales


def test_e4m3_values_derived_by_hand():
    # sign | exponent (bias 7) | mantissa: 0.0111.000 = 1, 0.0110.000 = 0.5, 1.1000.000 = -2,
    # 0.1111.110 = 1.75 * 2^8 = 448, 0.0001.000 = 2^-6 (smallest normal),
    # 0.0000.001 = 2^-9 (smallest subnormal), 0.0000.111 = 7 * 2^-9
    cases = {0x38: 1.0, 0x30: 0.5, 0xC0: -2.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0x3C: 1.5, 0x00: 0.0}
    for c, v in cases.items():
        assert O.e4m3_value(np.array([c]))[0] == v, hex(c)
    neg0 = O.e4m3_value(np.array([0x80]))[0]
    assert neg0 == 0.0 and np.signbit(neg0)
    assert np.isnan(O.e4m3_value(np.array([0x7F, 0xFF]))).all()
    assert np.isfinite(O.e4m3_value(np.array([0x7E, 0xFE]))).all()


def test_e4m3_values_match_torch_float8_e4m3fn():
    c = np.arange(256)
    mine = O.e4m3_value(c)
    ref = torch.tensor(c, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3_encode_round_trips_every_finite_code():
    c = np.array([x for x in range(256) if (x & 0x7F) != 0x7F])
    v = O.e4m3_value(c).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(v), c.astype(np.uint8))


def test_e4m3_encode_matches_torch_inside_the_range():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal(100000) * np.exp2(rng.uniform(-14, 9, 100000))).astype(np.float32)
    y = y[np.abs(y) <= 448]
    mine = O.e4m3_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_encode_ties_go_to_the_even_code_and_large_values_saturate():
    f = np.float32
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): the even code 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A): the even code 0x3A
    # 2^-10 lies halfway between 0 and 2^-9: code 0; 3 * 2^-10 between 0x01 and 0x02: 0x02
    # 1.9375 lies halfway between 1.875 (0x3F) and 2.0 (0x40): 0x40, the carry into the exponent
    ties = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 1.9375: 0x40,
            -1.0625: 0xB8, 0.015625 * 1.0625: 0x08}
    for y, c in ties.items():
        assert O.e4m3_encode(np.array([f(y)]))[0] == c, y
    for y in (448.0, 449.0, 464.0, 480.0, 1e30, np.finfo(np.float32).max):
        assert O.e4m3_encode(np.array([f(y)]))[0] == 0x7E
        assert O.e4m3_encode(np.array([f(-y)]))[0] == 0xFE
    assert O.e4m3_encode(np.array([f(-0.0)]))[0] == 0x80
    assert O.e4m3_encode(np.array([f(-2.0 ** -12)]))[0] == 0x80


def test_quantize_rows_invariants():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 256)).astype(np.float32) * np.exp2(rng.uniform(-6, 6, (64, 1))).astype(np.float32)
    codes, scales = O.e4m3_quantize_rows(x)
    amax = np.max(np.abs(x), axis=1)
    # the scale is the float32 quotient amax / 448
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    # the row's largest magnitude takes the largest code
    i = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(64), i]
    assert np.all((top & 0x7F) == 0x7E)
    # reconstruction error: half a code step, i.e. 2^-4 relative in the normal range, 2^-10 * scale below it
    deq = O.e4m3_dequantize(codes, scales)
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    # dequantization is exact: code x scale needs at most 4 + 24 significant bits
    v = O.e4m3_value(codes)
    assert np.array_equal(deq, v * scales[:, None].astype(np.float64))


def test_quantize_rows_special_rows():
    z = np.zeros((2, 256), np.float32)
    z[1, 7] = -0.0
    codes, scales = O.e4m3_quantize_rows(z)
    assert np.all(codes == 0) and np.all(scales == 0)
    # a row whose largest magnitude is 448 has scale 1 and is encoded as is
    r = np.linspace(-448, 448, 256, dtype=np.float32)
    c1, s1 = O.e4m3_quantize_rows(r[None])
    assert s1[0] == 1.0
    assert np.array_equal(c1[0], O.e4m3_encode(r))
    # a row of one value takes +-448 everywhere
    c2, s2 = O.e4m3_quantize_rows(np.full((1, 256), -3.25, np.float32))
    assert np.all(c2 == 0xFE) and s2[0] == np.float32(3.25) / np.float32(448)


def test_fp8_layout_offsets_by_hand():
    lay = O.PageLayout(n_kv_heads=2, head_dim=256, page_pos=4, dtype="fp8")
    # codes 2*4*256 = 2048 bytes each for K and V, scales 2*4*4 = 32 bytes each
    assert (lay.v_off, lay.ks_off, lay.vs_off, lay.page_bytes) == (2048, 4096, 4128, 4160)
    table = np.array([[3, 7]], np.int32)
    # scale of (s=0, h=1, p=5): page table[0][1] = 7, row 1*4 + 1 of 4-byte rows
    assert O.row_offset(table, 4, lay.page_elems, 0, 1, 5, 4) + lay.ks_off == 7 * 4160 + 4096 + 20
    # odd head x page_pos products are padded to 16 bytes
    assert O.PageLayout(1, 256, 3, "fp8").page_bytes == (6 * 256 + 24 + 15) // 16 * 16


@pytest.mark.parametrize("kind", ["reversed", "shuffled", None])
def test_fp8_place_gather_round_trip(kind):
    from paged_kv_cache_pg_amd.inputs import make_table
    rng = np.random.default_rng(3)
    lens = [9, 1, 16]
    ptok = 4 if kind else 16
    pages = [(l + ptok - 1) // ptok for l in lens]
    table, n_pages = make_table(kind, pages, rng)
    lay = O.PageLayout(2, 256, ptok, "fp8")
    KC = draw_e4m3_codes(rng, (3, 2, 16, 256))
    VC = draw_e4m3_codes(rng, (3, 2, 16, 256))
    KS = draw_row_scales(rng, (3, 2, 16))
    VS = draw_row_scales(rng, (3, 2, 16))
    arena = O.place_fp8(lay, table, n_pages, lens, KC, VC, KS, VS)
    kc, vc, ks, vs = O.gather_fp8(lay, table, arena, lens, cap=16)
    for s, L in enumerate(lens):
        assert np.array_equal(kc[s, :, :L], KC[s, :, :L]) and np.array_equal(vc[s, :, :L], VC[s, :, :L])
        assert np.array_equal(ks[s, :, :L], KS[s, :, :L]) and np.array_equal(vs[s, :, :L], VS[s, :, :L])


def test_generated_codes_are_never_nan_and_cover_the_range():
    c = draw_e4m3_codes(np.random.default_rng(0), 100000)
    assert not np.isin(c, [0x7F, 0xFF]).any()
    assert len(np.unique(c)) == 254
