"""Pins of the oracle's dense-and-sparse outlier quantization (one outlier per group)."""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import cache, layout, nbytes, quant

F32 = np.float32


def _by_sorting(x):
    """Outlier by a different route: stable sort of (-|x|) and take the first index."""
    return int(sorted(range(len(x)), key=lambda i: (-abs(Fraction(float(x[i]))), i))[0])


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("meta16", [False, True])
def test_outlier_is_exact_and_dense_range_excludes_it(bits, meta16):
    rng = np.random.default_rng(bits + 10 * meta16)
    for _ in range(50):
        kg = (rng.standard_normal((32, 6)) * rng.choice([0.1, 1, 10])).astype(np.float16)
        kg[rng.integers(32), rng.integers(6)] = np.float16(rng.choice([-300, 300, 60]))   # a planted outlier
        q, s, z, idx, val = quant.quantize_k_group(kg, bits, meta16, outliers=True)
        x = kg.astype(F32)
        for c in range(6):
            col = x[:, c]
            i = _by_sorting(col)
            assert idx[c] == i and val[c] == kg[i, c] and q[i, c] == 0
            rest = np.delete(col, i)
            # parameters equal those of the 31 others quantized on their own
            if meta16:
                s2, m2 = quant.int_group_params_f16(rest, bits, 0)
            else:
                s2, m2 = quant.int_group_params(rest, bits, 0)
            assert s[c] == s2 and z[c] == m2
        xh = quant.dequantize_k_group(q, s, z, idx, val)
        for c in range(6):
            i = idx[c]
            assert xh[i, c] == float(kg[i, c])                       # exact outlier
            others = np.delete(np.arange(32), i)
            bound = float(s[c]) * (0.5 + 2.0**-20 * ((1 << bits) + 2.0**16))
            assert np.all(np.abs(xh[others, c] - x[others, c]) <= bound)


def test_ties_take_the_lowest_index_and_signs_count_by_magnitude():
    x = np.array([[1.0, -7.0, 7.0, 2.0]], np.float16).astype(F32)
    assert quant.outlier_index(x, -1)[0] == 1
    y = np.array([[3.0, 3.0, -3.0]], np.float16).astype(F32)
    assert quant.outlier_index(y, -1)[0] == 0


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_grid_plus_one_outlier_reconstructs_exactly(bits):
    # 31 values on an exact grid (range exactly representable) plus one far value:
    # the dense part round-trips and the outlier is stored exactly, so x_hat == x
    qmax = (1 << bits) - 1
    s0 = 2.0**-6
    codes = np.arange(31) % (qmax + 1)
    codes[0], codes[1] = 0, qmax
    v = (s0 * (codes - 3)).astype(np.float16)
    v = np.concatenate([v[:10], np.array([np.float16(-50.0)]), v[10:]])[:, None].repeat(2, axis=1)
    q, s, z, idx, val = quant.quantize_k_group(v, bits, False, outliers=True)
    assert np.all(idx == 10) and np.all(s == F32(s0))
    assert np.array_equal(quant.dequantize_k_group(q, s, z, idx, val), v.astype(np.float64))
    # without the outlier split the same group loses resolution
    q2, s2, z2 = quant.quantize_k_group(v, bits)
    assert s2[0] > s[0]


@settings(max_examples=100, deadline=None)
@given(st.sampled_from([2, 4, 8]), st.booleans(),
       st.lists(st.floats(-6e4, 6e4, allow_nan=False, width=16), min_size=32, max_size=32))
def test_values_groups_bound(bits, meta16, vals):
    v = np.array(vals, np.float16)[None, :].repeat(2, axis=0)            # 2 tokens, D = 32, g_v = 32
    q, s, z, idx, val = quant.quantize_v_tokens(v, bits, 32, meta16, outliers=True)
    xh = quant.dequantize_v_tokens(q, s, z, idx, val)
    x = v.astype(np.float64)
    for t in range(2):
        i = idx[t, 0]
        assert xh[t, i] == x[t, i]
        assert i == _by_sorting(v[t].astype(F32))
        bound = float(s[t, 0]) * (0.5 + 2.0**-20 * ((1 << bits) + 2.0**16))
        assert np.all(np.abs(np.delete(xh[t], i) - np.delete(x[t], i)) <= bound)


def test_cache_with_outliers_and_layout():
    rng = np.random.default_rng(5)
    b, n, hkv, d = 1, 96, 2, 128
    k = rng.standard_normal((b, n, hkv, d)).astype(np.float16)
    v = rng.standard_normal((b, n, hkv, d)).astype(np.float16)
    k[0, 5, 1, 7] = np.float16(200.0)
    lay = cache.Layout(b, hkv, 2, d, n, "int4", residual_tokens=32, outliers=True)
    st_ = cache.build_cache(k, v, lay)
    assert st_.ko_idx.shape == (1, 2, 2, 128) and st_.vo_idx.shape == (1, 2, 64, 4)
    assert st_.ko_idx[0, 1, 0, 7] == 5 and st_.ko_val[0, 1, 0, 7] == np.float16(200.0)
    kh, vh = cache.dequantize(st_)
    assert kh[0, 1, 5, 7] == 200.0
    # entries round-trip through the documented 32-bit packing
    e = layout.pack_outliers(st_.ko_idx, st_.ko_val)
    assert e.dtype == np.uint32 and (int(e[0, 1, 0, 7]) & 0xFFFF) == 5
    i2, v2 = layout.unpack_outliers(e)
    assert np.array_equal(i2, st_.ko_idx) and np.array_equal(v2.view(np.uint16), st_.ko_val.view(np.uint16))
    ev = layout.pack_v_outliers(st_.vo_idx, st_.vo_val)
    assert ev.shape == (1, 2, 2, 4, 32)
    i3, v3 = layout.unpack_v_outliers(ev)
    assert np.array_equal(i3, st_.vo_idx) and np.array_equal(v3.view(np.uint16), st_.vo_val.view(np.uint16))
    # one 32-bit entry per 32-value group: one more bit per value
    sb0 = nbytes.step_bytes(cache.Layout(16, 8, 32, 128, 8192, "int4"), 8192)
    sb1 = nbytes.step_bytes(cache.Layout(16, 8, 32, 128, 8192, "int4", outliers=True), 8192)
    per_value = 8 * (sb1["meta"] - sb0["meta"]) / (2 * 16 * 8 * sb0["n_q"] * 128)
    assert per_value == 1.0
