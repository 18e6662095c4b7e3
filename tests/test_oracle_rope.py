"""Pins of the oracle's rotary position embedding and the pre-RoPE Key layout."""
import math

import numpy as np
import pytest

from oracle import attention as oattn
from oracle import cache, layout, rope


def test_rope_equals_complex_rotation():
    # pair (x_i, x_{i+D/2}) as the complex number x_i + j x_{i+D/2}, times e^{j pos theta_i}
    rng = np.random.default_rng(0)
    d, n = 128, 50
    x = rng.standard_normal((3, n, d))
    pos = rng.integers(0, 200000, size=n)
    for base in (10000.0, 500000.0):
        z = x[..., : d // 2] + 1j * x[..., d // 2:]
        i = np.arange(d // 2)
        zr = z * np.exp(1j * pos[:, None] * base ** (-2.0 * i / d))
        want = np.concatenate([zr.real, zr.imag], axis=-1)
        assert np.allclose(rope.apply_rope(x, pos, base), want, rtol=0, atol=1e-12)


def test_rope_closed_forms():
    # D = 2: theta_0 = 1 for any base, so position p rotates by p radians
    x = np.array([[1.0, 0.0]])
    for p in (0, 1, 3):
        assert np.allclose(rope.apply_rope(x, [p], 10000.0), [[math.cos(p), math.sin(p)]], atol=1e-15)
    # D = 4, base 10000: theta_1 = 10000^(-1/2) = 0.01, so position 100 rotates pair 1 by 1 radian
    y = np.array([[0.0, 2.0, 0.0, 0.0]])
    assert np.allclose(rope.apply_rope(y, [100], 10000.0), [[0.0, 2 * math.cos(1), 0.0, 2 * math.sin(1)]],
                       atol=1e-12)
    # position 0 is the identity; rotations keep every pair's length
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 128))
    assert np.array_equal(rope.apply_rope(z, np.zeros(5, int), 500000.0), z)
    r = rope.apply_rope(z, np.arange(5) * 977, 500000.0)
    assert np.allclose(np.hypot(r[:, :64], r[:, 64:]), np.hypot(z[:, :64], z[:, 64:]), rtol=1e-14)


def test_rope_logits_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(128)
    k = rng.standard_normal((20, 128))
    pk = rng.integers(0, 5000, size=20)
    for shift in (1, 37, 100000):
        a = rope.apply_rope(k, pk, 500000.0) @ rope.apply_rope(q[None], [6000], 500000.0)[0]
        b = rope.apply_rope(k, pk + shift, 500000.0) @ rope.apply_rope(q[None], [6000 + shift], 500000.0)[0]
        assert np.allclose(a, b, rtol=0, atol=1e-9)


def test_pre_rope_attention_is_rotated_attention():
    # a pre-RoPE cache attends with the rotated Keys; with rope_theta = 0 the Keys are used as stored
    rng = np.random.default_rng(3)
    b, n, hkv, d = 1, 96, 2, 128
    k = rng.standard_normal((b, n, hkv, d)).astype(np.float16)
    v = rng.standard_normal((b, n, hkv, d)).astype(np.float16)
    q = rng.standard_normal((b, 4, d))
    lay0 = cache.Layout(b, hkv, 4, d, n, "int8", residual_tokens=32)
    lay1 = cache.Layout(b, hkv, 4, d, n, "int8", residual_tokens=32, rope_theta=500000.0)
    st0, st1 = cache.build_cache(k, v, lay0), cache.build_cache(k, v, lay1)
    kh, vh = cache.dequantize(st1)
    assert np.array_equal(cache.attention_keys(st0, kh), kh)
    kr = cache.attention_keys(st1, kh)
    want = rope.apply_rope(kh, np.arange(n), 500000.0)
    assert np.array_equal(kr, want)
    out = oattn.attention(q, kr, vh)
    assert np.all(np.isfinite(out))


def test_stored_channel_pairs_are_adjacent():
    d = 128
    p = np.arange(d)
    ch = rope.stored_channel(p, d)
    assert sorted(ch) == list(range(d))
    assert np.all(ch[0::2] + d // 2 == ch[1::2]) and np.array_equal(ch[0::2], np.arange(d // 2))


@pytest.mark.parametrize("fmt,bits", [("int8", 8), ("int4", 4), ("int2", 2), ("fp8", 8)])
def test_pre_rope_k_layout(fmt, bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(2, 32, 128), dtype=np.uint8)
    plain = layout.pack_k_codes(codes, fmt)
    paired = layout.pack_k_codes(codes, fmt, rope=True)
    # the paired block is the plain block of the channel-permuted codes
    perm = rope.stored_channel(np.arange(128), 128)
    assert np.array_equal(paired, layout.pack_k_codes(codes[..., perm], fmt))
    assert not np.array_equal(paired, plain)
    assert np.array_equal(layout.unpack_k_codes(paired, fmt, 128, rope=True), codes)
    s = rng.standard_normal((2, 1, 128)).astype(np.float32)
    z = rng.standard_normal((2, 1, 128)).astype(np.float32)
    m = layout.pack_k_meta(s, z, rope=True)
    assert m[0, 0, 2 * 5 + 1, 0] == s[0, 0, 64 + 5] and m[0, 0, 2 * 5, 1] == z[0, 0, 5]
    s2, z2 = layout.unpack_k_meta(m, rope=True)
    assert np.array_equal(s2, s) and np.array_equal(z2, z)
