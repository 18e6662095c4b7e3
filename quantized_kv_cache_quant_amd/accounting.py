"""Algorithmic HBM bytes of one decode-attention call (for throughput reporting).

Counts what the method must move per layer and step, in this library's
layout: packed codes, scale / zero-point planes (INT formats: fp32 pairs, or
fp16 pairs with the fp16-metadata variant), the fp16
residual window and sinks, the fp16 query and the fp16 output.  Split-K
partials are implementation overhead and are not counted.  The KV_bytes
formula of "KV Cache Quantization Analysis" (memory-size sense box) is the
codes-only part of this count.
"""
from __future__ import annotations

BITS = {"int8": 8, "int4": 4, "int2": 2, "fp8": 8, "fp8_e5m2": 8}
BLOCK = 32


def routed(n: int, sink: int, residual: int):
    """(sinks, quantized body tokens, fp16 residual tokens) after n tokens."""
    ns = min(n, sink)
    body = n - ns
    nq = BLOCK * ((body - residual) // BLOCK) if body > residual else 0
    return ns, nq, body - nq


def attention_bytes(batch: int, kv_heads: int, q_heads: int, head_dim: int, n: int, fmt: str,
                    sink: int = 0, residual: int = 128, v_group: int = 32, meta_fp16: bool = False,
                    outliers: bool = False) -> int:
    ns, nq, r = routed(n, sink, residual)
    bh = batch * kv_heads
    codes = 2 * bh * nq * head_dim * BITS[fmt] // 8
    pair = (4 if meta_fp16 else 8) + (4 if outliers else 0)   # bytes per group: (s, z) pair + outlier entry
    meta = 0 if fmt.startswith("fp8") else (bh * (nq // BLOCK) * head_dim * pair
                                            + bh * nq * (head_dim // v_group) * pair)
    fp16 = 2 * bh * (ns + r) * head_dim * 2
    qo = 2 * batch * q_heads * head_dim * 2
    return codes + meta + fp16 + qo


def append_bytes(batch: int, kv_heads: int, head_dim: int, tokens: int = 1) -> int:
    """fp16 K and V read once per appended token (flushes excluded)."""
    return 2 * batch * kv_heads * tokens * head_dim * 2
