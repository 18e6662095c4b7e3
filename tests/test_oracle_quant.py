"""Pins of the oracle's quantization codecs against what the pages and IEEE fix.

Each test checks the oracle against something other than itself: printed
values, closed forms, exact rational arithmetic, exhaustive search, or a
library routine (torch's float8_e4m3fn cast).
"""
import json
import math
import os
from decimal import ROUND_HALF_UP, Decimal
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import nbytes, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


# ----------------------------------------------------------------- byte formula
def test_kv_bytes_70b_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "kv_size_70b.json")))
    sh = g["shape"]
    args = (sh["layers"], sh["kv_heads"], sh["head_dim"], sh["seq_len"], sh["batch"])
    bf16 = nbytes.kv_bytes(*args, g["bytes_per_element"]["fp16"])
    assert bf16 == 42_949_672_960 == 40 * 2**30           # "about 40 GB"
    for fmt, printed in g["printed_gb"].items():
        b = nbytes.kv_bytes(*args, nbytes.BYTES_PER_ELEM[fmt])
        assert b / 2**30 == printed                         # 40 / 20 / 10 (GiB)


def test_block_format_per_token_sizes():
    g = json.load(open(os.path.join(GOLDEN, "per_token_sizes_27b.json")))
    f = g["block_formats"]
    # the fp8 row fixes the number of cached values per token (8 bits, no scale)
    values = g["per_token_kib"]["fp8_e4m3"] * 1024 * 8 // 8
    for name, spec in f.items():
        bits = nbytes.block_bits_per_value(spec["bits"], spec["block"], spec["scale_bits"])
        per_token = values * bits / 8
        assert per_token == g["per_token_kib"][name] * 1024
        gib_64k = Decimal(per_token * 65536 / 2**30).quantize(Decimal("0.01"), ROUND_HALF_UP)
        assert str(gib_64k) == g["at_64k_gib_printed"][name]


# ------------------------------------------------------- fp32 rounding, exactly
def _rn32(fr: Fraction) -> np.float32:
    """Round a rational to the nearest float32, ties to even (independent of numpy ops)."""
    approx = np.float32(float(fr))
    cands = {approx, np.nextafter(approx, F32(np.inf)), np.nextafter(approx, F32(-np.inf))}
    best = sorted(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                        int(np.array(c, F32).view(np.uint32)) & 1))
    return best[0]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_group_params_are_rounded_exact_quotients(bits):
    rng = np.random.default_rng(7 + bits)
    for _ in range(200):
        x = (rng.standard_normal(32) * rng.choice([0.01, 1, 30])).astype(np.float16).astype(F32)
        s, z = quant.int_group_params(x, bits, axis=0)
        mn, mx = Fraction(float(x.min())), Fraction(float(x.max()))
        s_exp = _rn32((mx - mn) / ((1 << bits) - 1))
        if s_exp == 0:
            s_exp = F32(1.0)
        assert s == s_exp
        assert z == _rn32(-mn / Fraction(float(s_exp)))
        q = quant.int_encode(x, s, z, bits)
        for xi, qi in zip(x, q):
            a = _rn32(Fraction(float(xi)) / Fraction(float(s)))          # x / s
            v = _rn32(Fraction(float(a)) + Fraction(float(z)))           # + z
            # nearest code by exhaustive search, ties to the even code
            dist = [(abs(Fraction(float(v)) - c), c % 2, c) for c in range(1 << bits)]
            assert qi == min(dist)[2]


# ------------------------------------------------------------------ the s/2 bound
@settings(max_examples=150, deadline=None)
@given(st.integers(2, 8).filter(lambda b: b in (2, 4, 8)),
       st.lists(st.floats(-6e4, 6e4, allow_nan=False, width=16), min_size=1, max_size=64))
def test_error_bound_half_step(bits, vals):
    x = np.array(vals, np.float16).astype(F32)
    s, z = quant.int_group_params(x, bits, axis=0)
    q = quant.int_encode(x, s, z, bits)
    xh = quant.int_decode(q, s, z)
    bound = float(s) * (0.5 + 2.0**-20 * ((1 << bits) + abs(float(z))))
    assert np.all(np.abs(x.astype(np.float64) - xh) <= bound)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_grid_round_trip(bits):
    qmax = (1 << bits) - 1
    s0 = 2.0**-6
    for z0 in range(qmax + 1):
        codes = np.arange(qmax + 1)
        x = (s0 * (codes - z0)).astype(np.float16)
        assert np.all(x.astype(np.float64) == s0 * (codes - z0))     # on the fp16 grid
        perm = np.random.default_rng(z0).permutation(len(x))
        s, z = quant.int_group_params(x[perm].astype(F32), bits, axis=0)
        assert s == F32(s0) and z == F32(z0)
        q = quant.int_encode(x[perm].astype(F32), s, z, bits)
        assert np.array_equal(q, codes[perm])
        assert np.array_equal(quant.int_decode(q, s, z), x[perm].astype(np.float64))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_monotone_and_endpoints(bits):
    rng = np.random.default_rng(bits)
    for _ in range(100):
        x = (rng.standard_normal(32) * 3).astype(np.float16).astype(F32)
        s, z = quant.int_group_params(x, bits, axis=0)
        q = quant.int_encode(x, s, z, bits)
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(q[order].astype(int)) >= 0)
        if x.max() > x.min():
            assert q[np.argmin(x)] == 0 and q[np.argmax(x)] == (1 << bits) - 1


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_constant_group_is_exact(bits):
    for c in [0.0, -0.0, 1.5, -3.25, 65504.0]:
        x = np.full(32, c, np.float16).astype(F32)
        s, z = quant.int_group_params(x, bits, axis=0)
        q = quant.int_encode(x, s, z, bits)
        assert s == 1.0 and np.all(q == 0)
        assert np.all(quant.int_decode(q, s, z) == x.astype(np.float64))


def test_zero_minimum_gives_negative_zero_point():
    x = np.array([0.0, 1.0, 2.0, -0.0], np.float16).astype(F32)
    s, z = quant.int_group_params(x, 4, axis=0)
    assert np.signbit(z) and z == 0.0


# ------------------------------------------------------------------------ E4M3
def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = quant.e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0**-9 and tab[0x08] == 2.0**-6
    assert np.signbit(tab[0x80]) and tab[0x80] == 0.0


def test_e4m3_encode_decode_identity():
    tab = quant.e4m3_decode_table()
    finite = [c for c in range(256) if not np.isnan(tab[c])]
    assert np.array_equal(quant.e4m3_encode(tab[finite]), np.array(finite, np.uint8))


@pytest.mark.parametrize("scale", [1.0, 0.0078125, 0.013671875, 3.7, 146.28571])
def test_fp8_encode_matches_torch_cast(scale):
    s = F32(scale)
    x = np.arange(65536, dtype=np.uint16).view(np.float16)
    x = x[np.isfinite(x)]
    v = x.astype(F32) / s
    inside = np.abs(v) <= 448.0
    ours = quant.fp8_encode(x[inside], s)
    ref = torch.from_numpy(v[inside]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # outside the range the explicit clamp saturates to +-448
    out = quant.fp8_encode(x[~inside], s)
    assert np.all((out & 0x7F) == 0x7E)


def test_fp8_scale_recipe():
    x = np.array([[-3.0, 448.0 * 2]], np.float16)
    assert quant.fp8_scale(x) == F32(2.0)
    assert quant.fp8_scale(np.zeros(4, np.float16)) == F32(1.0)
    assert math.isclose(float(quant.fp8_decode(quant.fp8_encode(x, 2.0), 2.0)[0, 1]), 896.0)


# ------------------------------------------------------------------------ E5M2
def test_e5m2_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    tab = quant.e5m2_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    assert tab[0x7B] == 57344.0 and tab[0x7C] == np.inf and tab[0xFC] == -np.inf
    assert tab[0x01] == 2.0**-16 and np.signbit(tab[0x80])


def test_e5m2_is_the_top_byte_of_fp16():
    # E5M2 has fp16's sign and exponent fields and its two leading mantissa
    # bits, so code c is the fp16 with bit pattern c << 8
    tab = quant.e5m2_decode_table()
    h = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    both_nan = np.isnan(h) & np.isnan(tab)
    assert np.all(both_nan | (h == tab))


def test_e5m2_encode_decode_identity():
    tab = quant.e5m2_decode_table()
    finite = [c for c in range(256) if np.isfinite(tab[c])]
    assert np.array_equal(quant.e5m2_encode(tab[finite]), np.array(finite, np.uint8))


@pytest.mark.parametrize("scale", [1.0, 2.0**-20, 0.013671875, 3.7, 1.1428571])
def test_e5m2_encode_matches_torch_cast(scale):
    s = F32(scale)
    x = np.arange(65536, dtype=np.uint16).view(np.float16)
    x = x[np.isfinite(x)]
    v = x.astype(F32) / s
    inside = np.abs(v) <= 57344.0
    ours = quant.fp8_encode(x[inside], s, "fp8_e5m2")
    ref = torch.from_numpy(v[inside]).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    if np.any(~inside):
        out = quant.fp8_encode(x[~inside], s, "fp8_e5m2")
        assert np.all((out & 0x7F) == 0x7B)          # clamped to +-57344


def test_e5m2_scale_recipe():
    x = np.array([[-3.0, 28672.0]], np.float16)
    assert quant.fp8_scale(x, "fp8_e5m2") == F32(0.5)
    assert float(quant.fp8_decode(quant.fp8_encode(x, 0.5, "fp8_e5m2"), 0.5, "fp8_e5m2")[0, 1]) == 28672.0


# --------------------------------------------------- fp16 scale / offset metadata
def _f16_up_exact(fr: Fraction) -> np.float16:
    """Smallest fp16 >= fr, by search over all finite non-negative fp16 values."""
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    for h in pos:
        if Fraction(float(h)) >= fr:
            return h
    raise AssertionError("out of fp16 range")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_f16_params_and_codes_are_exact(bits):
    rng = np.random.default_rng(70 + bits)
    qmax = (1 << bits) - 1
    for _ in range(60):
        x = (rng.standard_normal(32) * rng.choice([0.01, 1, 30]) + rng.choice([0, 5, 900])).astype(
            np.float16).astype(F32)
        s, m = quant.int_group_params_f16(x, bits, axis=0)
        assert s.dtype == np.float16 and m.dtype == np.float16
        mn, mx = Fraction(float(x.min())), Fraction(float(x.max()))
        s32 = _rn32((mx - mn) / qmax)
        s_exp = _f16_up_exact(Fraction(float(s32))) if s32 != 0 else np.float16(1.0)
        assert s == s_exp and Fraction(float(m)) == mn
        q = quant.int_encode_offset(x, s, m, bits)
        for xi, qi in zip(x, q):
            d = _rn32(Fraction(float(xi)) - Fraction(float(m)))              # x - m
            v = _rn32(Fraction(float(d)) / Fraction(float(s)))               # / s
            dist = [(abs(Fraction(float(v)) - c), c % 2, c) for c in range(qmax + 1)]
            assert qi == min(dist)[2]


@settings(max_examples=150, deadline=None)
@given(st.integers(2, 8).filter(lambda b: b in (2, 4, 8)),
       st.lists(st.floats(-6e4, 6e4, allow_nan=False, width=16), min_size=1, max_size=64),
       st.sampled_from([0.0, 1000.0, -20000.0]))
def test_f16_error_bound_half_step(bits, vals, shift):
    x = (np.array(vals, np.float16).astype(F32) / F32(64) + F32(shift)).astype(np.float16).astype(F32)
    s, m = quant.int_group_params_f16(x, bits, axis=0)
    q = quant.int_encode_offset(x, s, m, bits)
    xh = quant.int_decode_offset(q, s, m)
    bound = float(s) * (0.5 + 2.0**-20 * (1 << bits))
    assert np.all(np.abs(x.astype(np.float64) - xh) <= bound)


def test_f16_offset_keeps_the_bound_where_an_f16_zero_point_would_not():
    # a narrow group far from zero: range 1 at 1500 gives z = -min / s close
    # to -22500, where fp16's spacing is 16, so an fp16 z would move the
    # grid by about 4 code steps; the fp16 offset m = min is exact
    x = (np.float16(1500.0) + np.arange(9, dtype=np.float16) * np.float16(0.125)).astype(F32)
    s32, z32 = quant.int_group_params(x, 4, axis=0)
    assert abs(float(np.float16(z32)) - float(z32)) > 3.5
    s, m = quant.int_group_params_f16(x, 4, axis=0)
    q = quant.int_encode_offset(x, s, m, 4)
    assert q[0] == 0 and q[-1] == 15
    assert np.max(np.abs(quant.int_decode_offset(q, s, m) - x)) <= float(s) / 2


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_f16_grid_round_trip(bits):
    qmax = (1 << bits) - 1
    s0 = 2.0**-6
    for m0 in [0.0, -1.5, 3.25, -0.015625 * qmax]:
        codes = np.arange(qmax + 1)
        x = (m0 + s0 * codes).astype(np.float16)
        assert np.all(x.astype(np.float64) == m0 + s0 * codes)        # on the fp16 grid
        perm = np.random.default_rng(bits).permutation(len(x))
        s, m = quant.int_group_params_f16(x[perm].astype(F32), bits, axis=0)
        assert s == np.float16(s0) and m == np.float16(m0)
        q = quant.int_encode_offset(x[perm].astype(F32), s, m, bits)
        assert np.array_equal(q, codes[perm])
        assert np.array_equal(quant.int_decode_offset(q, s, m), x[perm].astype(np.float64))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_f16_monotone_endpoints_constant(bits):
    rng = np.random.default_rng(bits + 40)
    for _ in range(100):
        x = (rng.standard_normal(32) * 3).astype(np.float16).astype(F32)
        s, m = quant.int_group_params_f16(x, bits, axis=0)
        q = quant.int_encode_offset(x, s, m, bits)
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(q[order].astype(int)) >= 0)
        if x.max() > x.min():
            assert q[np.argmin(x)] == 0 and q[np.argmax(x)] == (1 << bits) - 1
    for c in [0.0, -0.0, 1.5, -3.25, 65504.0]:
        x = np.full(32, c, np.float16).astype(F32)
        s, m = quant.int_group_params_f16(x, bits, axis=0)
        q = quant.int_encode_offset(x, s, m, bits)
        assert s == 1.0 and np.all(q == 0)
        assert np.all(quant.int_decode_offset(q, s, m) == x.astype(np.float64))


def test_f16_round_up_is_smallest_upper_bound():
    vals = np.array([0.0, 2.0**-30, 2.0**-24, 1.0, 1.0 + 2.0**-12, 1 / 3, 43669.0, 65504.0], F32)
    got = quant.f16_round_up(vals)
    for v, h in zip(vals, got):
        assert h == _f16_up_exact(Fraction(float(v)))
