"""The library's byte layout of the packed cache, restated for comparison.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages fix no byte layout: they only say that codes, scales and
zero-points are stored (scale storage eats part of the saving, "KV Cache
Quantization Analysis", sec. 2 granularity bullet) and that the recent
window stays in full precision (sec. 3).  The layout below is the one the
library documents in ``include/kvq.h``; this module writes it out
independently so that tests can compare the library's planes byte for byte.

Planes (per layer; NB = quantized blocks of 32 tokens, b = bits per code):

* K codes   [B][Hkv][NB][32*D*b/8]  the codes of one token are D*b/8 bytes,
  channel c at bit (c*b mod 8) of byte floor(c*b/8) (LSB first; FP8: one
  byte per code).  INT4 / INT2: the 32 tokens' byte rows one after another.
  INT8 / FP8: 16-byte units; unit u = (2*tile + half)*(D/2) + 16*qd + r holds
  bytes 32*qd + 16*half .. +15 of token 16*tile + r.
* V codes   [B][Hkv][NB][32*D*b/8]  one block of 32 tokens is 64 "records"
  of D*b/16 bytes, split into 16-byte groups; group i of record l is stored
  at byte 16*(64*i + l).  Record l = 16*qd + r holds channels {16*m + r} for
  m = 0 .. D/16-1 and the eight tokens T = (4qd, 4qd+1, 4qd+2, 4qd+3,
  16+4qd, 16+4qd+1, 16+4qd+2, 16+4qd+3) of the block, laid out per format:
    INT4  word m: nibble j (bits 4j..4j+3) = code(T[j], 16m + r)
    INT8, FP8  bytes 8m .. 8m+7 = codes of T[0], T[4], T[1], T[5], T[2],
          T[6], T[3], T[7] for channel 16m + r
    INT2  word p (channels 16*(2p) + r = "A" and 16*(2p+1) + r = "B"):
          byte 0 = A's T[0..3], byte 1 = B's T[0..3], byte 2 = A's T[4..7],
          byte 3 = B's T[4..7], two bits per code, LSB first.
* K meta    [B][Hkv][NB][D][2]        fp32: (s, z) of each channel of the block's group
* V meta    [B][Hkv][NB][D/G_v][32][2] fp32: (s, z) of each channel group and token
  (fp16 metadata: the same shapes holding fp16 (s, m) pairs, m the offset)
* K / V ring   [B][Hkv][R+32][D] fp16;  K / V sinks  [B][Hkv][S][D] fp16.

Caches with dense-and-sparse outliers add two planes of 32-bit entries, the
index in the group in the low 16 bits and the fp16 value in the high 16:
K outliers [NB][D] (token index of each channel's outlier in the block) and
V outliers [NB][D/G_v][32] (channel index in the group, per group and token,
the V meta order).

Caches that store the Keys before RoPE keep each K row (codes and the K
meta plane alike) in RoPE pair order: stored position 2i holds channel i and
2i + 1 holds channel i + D/2, so each rotated pair sits side by side.

Paged caches keep the four quantized planes as a pool of pages, each page
P consecutive 32-token blocks of one sequence for all KV heads: records
ordered [page][Hkv][P].  Logical block j of (sequence b, head h) is record
(table[b][j // P] * Hkv + h) * P + j % P ("Quantization and the KV cache:
two ways to run a model lighter", KV-cache side: small blocks and a table
per request; "KV Cache Quantization Analysis", sec. 5: paging is orthogonal
to quantization).
"""
from __future__ import annotations

import numpy as np

from .rope import stored_channel

BLOCK = 32


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack the last axis of ``codes`` LSB-first: element i at bit i*b."""
    codes = np.asarray(codes, np.uint8)
    if bits == 8:
        return codes.copy()
    per = 8 // bits
    n = codes.shape[-1]
    assert n % per == 0
    c = codes.reshape(codes.shape[:-1] + (n // per, per)).astype(np.uint16)
    shifts = (np.arange(per) * bits).astype(np.uint16)
    return np.bitwise_or.reduce(c << shifts, axis=-1).astype(np.uint8)


def unpack_bits(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Inverse of :func:`pack_bits` (``n`` codes along the last axis)."""
    packed = np.asarray(packed, np.uint8)
    if bits == 8:
        return packed[..., :n].copy()
    per = 8 // bits
    shifts = (np.arange(per) * bits).astype(np.uint8)
    c = (packed[..., :, None] >> shifts) & ((1 << bits) - 1)
    return c.reshape(packed.shape[:-1] + (packed.shape[-1] * per,))[..., :n].astype(np.uint8)


def _record_tokens(qd: int):
    return [4 * qd + j for j in range(4)] + [16 + 4 * qd + j for j in range(4)]


def _v_record_order(fmt: str, d: int):
    """(token, channel) of every code of a V block, record after record."""
    if d % 32:
        raise ValueError("head_dim must be a multiple of 32")
    tok, ch = [], []
    sigma = [0, 4, 1, 5, 2, 6, 3, 7]
    for lane in range(64):
        qd, r = divmod(lane, 16)
        t = _record_tokens(qd)
        if fmt == "int4":
            for m in range(d // 16):
                for j in range(8):
                    tok.append(t[j]); ch.append(16 * m + r)
        elif fmt in ("int8", "fp8", "fp8_e5m2"):
            for m in range(d // 16):
                for k in range(8):
                    tok.append(t[sigma[k]]); ch.append(16 * m + r)
        elif fmt == "int2":
            for p in range(d // 32):
                for tile, half in ((2 * p, 0), (2 * p + 1, 0), (2 * p, 4), (2 * p + 1, 4)):
                    for j in range(4):
                        tok.append(t[half + j]); ch.append(16 * tile + r)
        else:
            raise ValueError(fmt)
    return np.array(tok), np.array(ch)


def _group_major(order: np.ndarray, bits: int) -> np.ndarray:
    """Reorder a 64-record stream so 16-byte group i of record l comes at 64*i + l."""
    per16 = 16 * 8 // bits                          # codes per 16 bytes
    return order.reshape(64, -1, per16).transpose(1, 0, 2).reshape(-1)


def v_block_stream_order(fmt: str, d: int):
    """(token, channel) of every code of a V block in packed-stream order."""
    tok, ch = _v_record_order(fmt, d)
    bits = _bits(fmt)
    return _group_major(tok, bits), _group_major(ch, bits)


def k_block_stream_order(fmt: str, d: int):
    """(token, channel) of every code of a K block in packed-stream order."""
    bits = _bits(fmt)
    if bits < 8:
        return np.repeat(np.arange(BLOCK), d), np.tile(np.arange(d), BLOCK)
    if d % 32:
        raise ValueError("head_dim must be a multiple of 32")
    tok, ch = [], []
    for tile in range(BLOCK // 16):
        for half in range(2):
            for lane in range(d // 2):
                qd, r = divmod(lane, 16)
                for e in range(16):
                    tok.append(16 * tile + r); ch.append(32 * qd + 16 * half + e)
    return np.array(tok), np.array(ch)


def _bits(fmt: str) -> int:
    return {"int8": 8, "int4": 4, "int2": 2, "fp8": 8, "fp8_e5m2": 8}[fmt]


def _pack_blocks(codes: np.ndarray, fmt: str, order) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    n, d = codes.shape[-2:]
    assert n % BLOCK == 0
    blk = codes.reshape(codes.shape[:-2] + (n // BLOCK, BLOCK, d))
    tok, ch = order(fmt, d)
    return pack_bits(blk[..., tok, ch], _bits(fmt))


def _unpack_blocks(packed: np.ndarray, fmt: str, d: int, order) -> np.ndarray:
    packed = np.asarray(packed, np.uint8)
    nb = packed.shape[-2]
    stream = unpack_bits(packed, _bits(fmt), BLOCK * d)
    tok, ch = order(fmt, d)
    out = np.zeros(packed.shape[:-1] + (BLOCK, d), np.uint8)
    out[..., tok, ch] = stream
    return out.reshape(packed.shape[:-2] + (nb * BLOCK, d))


def _to_stored(x: np.ndarray, rope: bool) -> np.ndarray:
    """Channel axis (last) in stored order: RoPE pair order for pre-RoPE caches."""
    x = np.asarray(x)
    return x[..., stored_channel(np.arange(x.shape[-1]), x.shape[-1])] if rope else x


def _from_stored(x: np.ndarray, rope: bool) -> np.ndarray:
    x = np.asarray(x)
    if not rope:
        return x
    out = np.empty_like(x)
    out[..., stored_channel(np.arange(x.shape[-1]), x.shape[-1])] = x
    return out


def pack_k_codes(codes: np.ndarray, fmt: str, rope: bool = False) -> np.ndarray:
    """[..., NB*32, D] codes -> [..., NB, 32*D*b/8] K block bytes."""
    return _pack_blocks(_to_stored(codes, rope), fmt, k_block_stream_order)


def unpack_k_codes(packed: np.ndarray, fmt: str, d: int, rope: bool = False) -> np.ndarray:
    """Inverse of :func:`pack_k_codes`: [..., NB, bytes] -> [..., NB*32, D]."""
    return _from_stored(_unpack_blocks(packed, fmt, d, k_block_stream_order), rope)


def pack_v_codes(codes: np.ndarray, fmt: str) -> np.ndarray:
    """[..., NB*32, D] codes -> [..., NB, 32*D*b/8] swizzled V block bytes."""
    return _pack_blocks(codes, fmt, v_block_stream_order)


def unpack_v_codes(packed: np.ndarray, fmt: str, d: int) -> np.ndarray:
    """Inverse of :func:`pack_v_codes`: [..., NB, bytes] -> [..., NB*32, D]."""
    return _unpack_blocks(packed, fmt, d, v_block_stream_order)


def _meta_dtype(s):
    """fp16 metadata stays fp16 (the fp16 (s, m) variant); anything else is fp32."""
    return np.float16 if np.asarray(s).dtype == np.float16 else np.float32


def pack_k_meta(s: np.ndarray, z: np.ndarray, rope: bool = False) -> np.ndarray:
    """s, z [..., NB, D] -> [..., NB, D, 2] (interleaved pairs, fp32 or fp16; stored order)."""
    dt = _meta_dtype(s)
    return np.stack([_to_stored(np.asarray(s, dt), rope), _to_stored(np.asarray(z, dt), rope)], axis=-1)


def pack_v_meta(s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """s, z [..., NB*32, Gn] -> [..., NB, Gn, 32, 2] (interleaved pairs, fp32 or fp16)."""
    dt = _meta_dtype(s)
    s = np.asarray(s, dt)
    z = np.asarray(z, dt)
    n, gn = s.shape[-2:]
    nb = n // BLOCK
    sb = np.swapaxes(s.reshape(s.shape[:-2] + (nb, BLOCK, gn)), -1, -2)
    zb = np.swapaxes(z.reshape(z.shape[:-2] + (nb, BLOCK, gn)), -1, -2)
    return np.stack([sb, zb], axis=-1)


def unpack_k_meta(m: np.ndarray, rope: bool = False):
    """[..., NB, D, 2] -> s, z [..., NB, D] (channel order)."""
    m = np.asarray(m, _meta_dtype(m))
    return _from_stored(m[..., 0], rope).copy(), _from_stored(m[..., 1], rope).copy()


def unpack_v_meta(m: np.ndarray):
    """[..., NB, Gn, 32, 2] -> s, z [..., NB*32, Gn]."""
    m = np.asarray(m, _meta_dtype(m))
    nb, gn, blk, _ = m.shape[-4:]
    s = np.swapaxes(m[..., 0], -1, -2).reshape(m.shape[:-4] + (nb * blk, gn))
    z = np.swapaxes(m[..., 1], -1, -2).reshape(m.shape[:-4] + (nb * blk, gn))
    return s.copy(), z.copy()


def paged_record(table: np.ndarray, b: int, h: int, blk: int, hkv: int, page_blocks: int) -> int:
    """Pool record holding logical block ``blk`` of (sequence b, head h)."""
    page = int(table[b, blk // page_blocks])
    return (page * hkv + h) * page_blocks + blk % page_blocks


def gather_paged(pool: np.ndarray, table: np.ndarray, hkv: int, page_blocks: int, nb: int) -> np.ndarray:
    """Pool records [n_records, ...] -> logical blocks [B, Hkv, nb, ...] through the table."""
    pool = np.asarray(pool)
    table = np.asarray(table, np.int64)
    b = table.shape[0]
    blk = np.arange(nb)
    page = table[:, blk // page_blocks]                           # [B, nb]
    rec = (page[:, None, :] * hkv + np.arange(hkv)[None, :, None]) * page_blocks + (blk % page_blocks)[None, None]
    return pool[rec.reshape(-1)].reshape((b, hkv, nb) + pool.shape[1:])


def pack_outliers(idx: np.ndarray, val: np.ndarray) -> np.ndarray:
    """Outlier entries: index | fp16 bits << 16, as uint32."""
    bits = np.asarray(val, np.float16).view(np.uint16).astype(np.uint32)
    return (np.asarray(idx).astype(np.uint32) | (bits << 16)).astype(np.uint32)


def unpack_outliers(e: np.ndarray):
    """Inverse of :func:`pack_outliers`: (index int64, value fp16)."""
    e = np.asarray(e, np.uint32)
    return (e & 0xFFFF).astype(np.int64), (e >> 16).astype(np.uint16).view(np.float16)


def pack_v_outliers(idx: np.ndarray, val: np.ndarray) -> np.ndarray:
    """[..., NB*32, Gn] -> [..., NB, Gn, 32] entries (group-major like the V meta)."""
    e = pack_outliers(idx, val)
    n, gn = e.shape[-2:]
    return np.swapaxes(e.reshape(e.shape[:-2] + (n // BLOCK, BLOCK, gn)), -1, -2)


def unpack_v_outliers(e: np.ndarray):
    """[..., NB, Gn, 32] -> index, value [..., NB*32, Gn]."""
    e = np.asarray(e, np.uint32)
    nb, gn, blk = e.shape[-3:]
    t = np.swapaxes(e, -1, -2).reshape(e.shape[:-3] + (nb * blk, gn))
    return unpack_outliers(t)
