"""Pins of the oracle's restatement of the library's byte layout.

The forward formulas below locate each code from the plain-language layout
rules (record, word, nibble) one element at a time; the oracle builds the
layout from a stream order.  Agreement pins the stream order.
"""
import numpy as np
import pytest

from oracle import layout


def _tok(qd, j):
    return 4 * qd + j if j < 4 else 16 + 4 * qd + (j - 4)


@pytest.mark.parametrize("fmt,bits", [("int4", 4), ("int8", 8), ("fp8", 8), ("fp8_e5m2", 8), ("int2", 2)])
def test_v_block_layout_rules(fmt, bits):
    rng = np.random.default_rng(bits)
    d = 128
    codes = rng.integers(0, 1 << bits, size=(2, 32, d), dtype=np.uint8)
    if fmt == "fp8":
        codes = rng.integers(0, 256, size=(2, 32, d), dtype=np.uint8)
    packed = layout.pack_v_codes(codes.reshape(64, d), fmt)          # [2 blocks][bytes]
    assert packed.shape == (2, 32 * d * bits // 8)
    sigma = [0, 4, 1, 5, 2, 6, 3, 7]
    for blk in range(2):
        for lane in range(64):
            qd, r = divmod(lane, 16)

            def at(x):                            # byte x of record `lane`
                i, e = divmod(x, 16)
                return int(packed[blk, 16 * (64 * i + lane) + e])
            for m in range(d // 16):
                ch = 16 * m + r
                for j in range(8):
                    t = _tok(qd, j)
                    c = codes[blk, t, ch]
                    if fmt == "int4":
                        word = sum(at(4 * m + i) << (8 * i) for i in range(4))
                        assert (word >> (4 * j)) & 0xF == c
                    elif bits == 8:
                        k = sigma.index(j)
                        assert at(8 * m + k) == c
                    else:
                        p, tile_b = divmod(m, 2)
                        byte = (2 if j >= 4 else 0) + tile_b
                        jj = j % 4
                        assert (at(4 * p + byte) >> (2 * jj)) & 3 == c
    assert np.array_equal(layout.unpack_v_codes(packed, fmt, d), codes.reshape(64, d))


@pytest.mark.parametrize("bits,fmt", [(2, "int2"), (4, "int4"), (8, "int8"), (8, "fp8")])
def test_k_block_layout_rules(bits, fmt):
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 1 << bits, size=(3, 64, 128), dtype=np.uint8)
    packed = layout.pack_k_codes(codes, fmt)
    assert packed.shape == (3, 2, 32 * 128 * bits // 8)
    row = 128 * bits // 8
    for blk in range(2):
        for t in range(32):
            for c in range(128):
                if bits == 8:                      # unit (tile, half, 16 qd + r), byte e
                    tile, r = divmod(t, 16)
                    qd, rest = divmod(c, 32)
                    half, e = divmod(rest, 16)
                    off = ((2 * tile + half) * 64 + 16 * qd + r) * 16 + e
                    got = packed[:, blk, off]
                else:                              # token rows, LSB first
                    byte, bit = divmod(c * bits, 8)
                    got = (packed[:, blk, t * row + byte] >> bit) & ((1 << bits) - 1)
                assert np.array_equal(got, codes[:, 32 * blk + t, c])
    assert np.array_equal(layout.unpack_k_codes(packed, fmt, 128), codes)


def test_meta_layouts():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((2, 3, 128)).astype(np.float32)
    z = rng.standard_normal((2, 3, 128)).astype(np.float32)
    m = layout.pack_k_meta(s, z)
    assert m.shape == (2, 3, 128, 2) and np.array_equal(m[..., 1], z)
    flat = m.reshape(2, 3, 256)                       # (s, z) pairs per channel
    assert flat[1, 2, 2 * 77] == s[1, 2, 77] and flat[1, 2, 2 * 77 + 1] == z[1, 2, 77]
    s2, z2 = layout.unpack_k_meta(m)
    assert np.array_equal(s2, s) and np.array_equal(z2, z)
    sv = rng.standard_normal((2, 64, 4)).astype(np.float32)
    zv = rng.standard_normal((2, 64, 4)).astype(np.float32)
    mv = layout.pack_v_meta(sv, zv)
    assert mv.shape == (2, 2, 4, 32, 2)
    flat = mv.reshape(2, 2, 256)                      # block: [group][token][s, z]
    assert flat[1, 1, 2 * (3 * 32 + 7)] == sv[1, 32 + 7, 3]
    assert flat[0, 0, 2 * (2 * 32 + 31) + 1] == zv[0, 31, 2]
    s2, z2 = layout.unpack_v_meta(mv)
    assert np.array_equal(s2, sv) and np.array_equal(z2, zv)
    # fp16 (s, m) metadata keeps its type: 4-byte pairs in the same order
    s16, m16 = s.astype(np.float16), z.astype(np.float16)
    m = layout.pack_k_meta(s16, m16)
    assert m.dtype == np.float16 and m.shape == (2, 3, 128, 2)
    assert m.reshape(2, 3, 256)[1, 2, 2 * 77 + 1] == m16[1, 2, 77]
    s2, z2 = layout.unpack_k_meta(m)
    assert s2.dtype == np.float16 and np.array_equal(s2, s16) and np.array_equal(z2, m16)
    mv = layout.pack_v_meta(sv.astype(np.float16), zv.astype(np.float16))
    assert mv.dtype == np.float16 and mv.reshape(2, 2, 256)[1, 1, 2 * (3 * 32 + 7)] == np.float16(sv[1, 32 + 7, 3])


@pytest.mark.parametrize("fmt", ["int8", "int4", "int2", "fp8"])
def test_empty_planes_unpack(fmt):
    bits = {"int8": 8, "int4": 4, "int2": 2, "fp8": 8}[fmt]
    k = layout.unpack_k_codes(np.zeros((2, 3, 0, 32 * 128 * bits // 8), np.uint8), fmt, 128)
    assert k.shape == (2, 3, 0, 128)
    v = layout.unpack_v_codes(np.zeros((2, 3, 0, 32 * 128 * bits // 8), np.uint8), fmt, 128)
    assert v.shape == (2, 3, 0, 128)


@pytest.mark.parametrize("page_blocks", [1, 3])
def test_paged_gather_follows_the_record_rule(page_blocks):
    rng = np.random.default_rng(page_blocks)
    b, hkv, nb = 3, 2, 7
    pages_per_seq = -(-nb // page_blocks)
    num_pages = b * pages_per_seq + 4
    table = rng.permutation(num_pages)[:b * pages_per_seq].reshape(b, pages_per_seq)
    pool = rng.integers(0, 256, size=(num_pages * hkv * page_blocks, 5), dtype=np.uint8)
    got = layout.gather_paged(pool, table, hkv, page_blocks, nb)
    assert got.shape == (b, hkv, nb, 5)
    for bi in range(b):
        for h in range(hkv):
            for j in range(nb):
                # page = table[b][j // P]; records ordered [page][Hkv][P]
                page = table[bi, j // page_blocks]
                rec = page * hkv * page_blocks + h * page_blocks + j % page_blocks
                assert layout.paged_record(table, bi, h, j, hkv, page_blocks) == rec
                assert np.array_equal(got[bi, h, j], pool[rec])
    # distinct pages give distinct records: the logical blocks are a permutation of pool rows
    recs = {layout.paged_record(table, bi, h, j, hkv, page_blocks)
            for bi in range(b) for h in range(hkv) for j in range(nb)}
    assert len(recs) == b * hkv * nb
