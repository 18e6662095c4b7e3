"""Seeded synthetic inputs for the quantized KV cache (no method arithmetic).

The pages measure on models and datasets that are not available here
(WikiText-2, GSM8K, LongBench, a 64k-token KL-divergence set).  These
generators stand in for them with the shapes of the Llama-3 layers the pages
use and the structure they describe: Key caches with a few fixed channels of
large magnitude ("KV Cache Quantization Analysis", sec. 3), attention-sink
tokens with dominant logits ("W4A16 + KV cache quantization: combined
accuracy", layer-sensitivity section).

Recipe: ``numpy.random.default_rng(seed).standard_normal(dtype=float32)``,
multiplied by the outlier / sink factors in fp32, then cast to fp16 (round
to nearest even).  Outlier channels are fixed across batch and tokens.
Both the oracle side of the tests and the GPU side receive the same arrays.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload (one decoder layer shape)."""
    name: str
    index: int                      # seeds: K 1000+i, V 2000+i, q 3000+i, outliers 4000+i
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int
    formats: tuple                  # per-layer format list, or one format per variant
    layers: int = 1
    residual_tokens: int = 128
    sink_tokens: int = 0
    k_group_tokens: int = 32
    v_group_channels: int = 32
    outlier_channels: int = 0       # count of (kv head, channel) pairs
    outlier_factor: float = 1.0
    sink_factor: float = 1.0
    append_steps: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, batch=1, num_q_heads=4, num_kv_heads=1, head_dim=128, seq_len=256,
        formats=("int4",), residual_tokens=32, outlier_channels=4, outlier_factor=10.0,
        notes="batch 1, 4 q heads on 1 KV head, seq 256, K/V INT4, residual 32"),
    "llama3_8b": Workload(
        "llama3_8b", 2, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_len=8192,
        formats=("fp8", "int8"), layers=32, outlier_channels=10, outlier_factor=20.0,
        notes="Llama-3-8B layer shape, batch 16, seq 8192, FP8 E4M3 or INT8 K/V"),
    "llama3_8b_kivi2": Workload(
        "llama3_8b_kivi2", 3, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_len=8192, formats=("int2",), layers=32, outlier_channels=10, outlier_factor=20.0,
        append_steps=64,
        notes="Llama-3-8B layer shape, INT2 K per-channel / V per-token, append 1 token/step"),
    "llama3_70b": Workload(
        "llama3_70b", 4, batch=16, num_q_heads=64, num_kv_heads=8, head_dim=128, seq_len=8192,
        formats=("int4",), layers=80, sink_tokens=4, sink_factor=10.0,
        notes="Llama-3-70B layer shape, INT4, 4 fp16 sink tokens with 10x K"),
    "long_ctx": Workload(
        "long_ctx", 5, batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_len=131072,
        formats=tuple(["int8"] * 4 + ["int4"] * 24 + ["int8"] * 4), layers=32,
        outlier_channels=10, outlier_factor=20.0,
        notes="batch 1, seq 131072, layers 0-3 and 28-31 INT8, 4-27 INT4"),
}


def outlier_pairs(w: Workload, num_kv_heads: int | None = None, head_dim: int | None = None):
    """(kv_head, channel) pairs that carry the fixed K outliers (seed 4000+i)."""
    hkv = num_kv_heads or w.num_kv_heads
    d = head_dim or w.head_dim
    if w.outlier_channels == 0:
        return np.zeros((0, 2), np.int64)
    rng = np.random.default_rng(4000 + w.index)
    flat = rng.choice(hkv * d, size=min(w.outlier_channels, hkv * d), replace=False)
    return np.stack([flat // d, flat % d], axis=1).astype(np.int64)


def kv_tokens(w: Workload, seed_k: int, seed_v: int, batch: int, tokens: int,
              num_kv_heads: int | None = None, head_dim: int | None = None,
              first_token: int = 0):
    """fp16 K, V of shape [batch][tokens][Hkv][D] for absolute tokens first_token.."""
    hkv = num_kv_heads or w.num_kv_heads
    d = head_dim or w.head_dim
    shape = (batch, tokens, hkv, d)
    k = np.random.default_rng(seed_k).standard_normal(shape, dtype=np.float32)
    v = np.random.default_rng(seed_v).standard_normal(shape, dtype=np.float32)
    pairs = outlier_pairs(w, hkv, d)
    if len(pairs):
        k[:, :, pairs[:, 0], pairs[:, 1]] *= np.float32(w.outlier_factor)
    if w.sink_tokens and first_token < w.sink_tokens:
        last = min(tokens, w.sink_tokens - first_token)
        k[:, :last] *= np.float32(w.sink_factor)
    return k.astype(np.float16), v.astype(np.float16)


def prefill(w: Workload, batch: int | None = None, tokens: int | None = None,
            num_kv_heads: int | None = None, head_dim: int | None = None):
    """The prompt's K, V (seeds 1000+i, 2000+i)."""
    return kv_tokens(w, 1000 + w.index, 2000 + w.index, batch or w.batch,
                     tokens or w.seq_len, num_kv_heads, head_dim)


def append_step(w: Workload, step: int, batch: int | None = None,
                num_kv_heads: int | None = None, head_dim: int | None = None,
                first_token: int | None = None):
    """K, V of the single token appended at decode step ``step`` (seed 5000+100i+j).

    The token's absolute position defaults to seq_len + step (after the prompt).
    """
    s = 5000 + 100 * w.index + step
    pos = w.seq_len + step if first_token is None else first_token
    return kv_tokens(w, s, s + 50, batch or w.batch, 1, num_kv_heads, head_dim, first_token=pos)


def queries(w: Workload, batch: int | None = None, num_q_heads: int | None = None,
            head_dim: int | None = None, seed_offset: int = 0):
    """fp16 decode queries [batch][Hq][D] (seed 3000+i)."""
    shape = (batch or w.batch, num_q_heads or w.num_q_heads, head_dim or w.head_dim)
    q = np.random.default_rng(3000 + w.index + seed_offset).standard_normal(shape, dtype=np.float32)
    return q.astype(np.float16)
