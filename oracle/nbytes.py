"""Byte accounting of the KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* :func:`kv_bytes` is the "memory-size sense" box of "KV Cache Quantization
  Analysis": KV_bytes = 2 x layers x kv_heads x head_dim x seq_len x batch x
  bytes per element, with FP16 = 2, FP8/INT8 = 1, INT4 = 0.5, INT2 = 0.25.
  "W4A16 + KV cache quantization: combined accuracy" works it for the 70B
  shape (80 layers, 8 KV heads, head_dim 128, batch 16, seq 8192): about
  40 GB at BF16, 20 GB at FP8, 10 GB at INT4.
* :func:`block_bits_per_value` counts block-quantized formats that keep one
  16-bit scale per block of values (the community 27B study prints per-token
  sizes 34 KiB for 8-bit q8_0 / EXL3, 32 KiB for fp8_e4m3 and 18 KiB for 4-bit
  q4_0 / EXL3, i.e. 8.5 : 8 : 4.5 bits per value).
* :func:`step_bytes` is the algorithmic HBM traffic of one decode step of one
  layer in this library's layout: packed codes + scale/zero planes (fp32, or
  fp16 with the fp16-metadata variant) +
  fp16 residual window + fp16 sinks + the fp16 query + the fp16 output.
"""
from __future__ import annotations

from .cache import Layout, window_split

BYTES_PER_ELEM = {"fp16": 2.0, "bf16": 2.0, "fp8": 1.0, "fp8_e5m2": 1.0, "int8": 1.0, "int4": 0.5,
                  "int2": 0.25}


def kv_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, batch: int,
             bytes_per_elem: float) -> float:
    """2 x L x n_kv_heads x head_dim x seq_len x batch x bytes (metadata excluded)."""
    return 2 * layers * kv_heads * head_dim * seq_len * batch * bytes_per_elem


def block_bits_per_value(code_bits: int, block: int, scale_bits: int) -> float:
    """Bits per value of a block format with one scale of ``scale_bits`` per ``block``."""
    return code_bits + scale_bits / block


def step_bytes(lay: Layout, n: int) -> dict:
    """Algorithmic bytes one decode-attention step reads and writes for one layer.

    ``n`` is the number of cached tokens (after the step's append).  Returns a
    dict with the parts and their ``total``.
    """
    b, hkv, hq, d = lay.batch, lay.num_kv_heads, lay.num_q_heads, lay.head_dim
    n_sink, n_q, r = window_split(n, lay.sink_tokens, lay.residual_tokens, lay.k_group_tokens)
    codes = 2 * b * hkv * n_q * d * lay.bits // 8
    if lay.fmt in ("fp8", "fp8_e5m2"):
        meta = 0
    else:
        eb = 2 if lay.meta_fp16 else 4                 # bytes per scale / zero-point
        meta_k = b * hkv * (n_q // lay.k_group_tokens) * d * 2 * eb
        meta_v = b * hkv * n_q * (d // lay.v_group_channels) * 2 * eb
        if lay.outliers:                               # one 4-byte entry per group
            meta_k += b * hkv * (n_q // lay.k_group_tokens) * d * 4
            meta_v += b * hkv * n_q * (d // lay.v_group_channels) * 4
        meta = meta_k + meta_v
    fp16 = 2 * b * hkv * (r + n_sink) * d * 2
    qo = 2 * b * hq * d * 2
    return {"codes": codes, "meta": meta, "fp16": fp16, "q_out": qo,
            "total": codes + meta + fp16 + qo, "n_q": n_q, "r": r, "n_sink": n_sink}
