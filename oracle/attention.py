"""fp64 decode attention over the dequantized cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"W4A16 + KV cache quantization: combined accuracy", section on where the
errors meet, writes the attention score as softmax(Q K^T / sqrt(d)); the
same page's worked example uses GQA with 8 KV heads shared by the query
heads.  "KV Cache Quantization Analysis", sec. 5, has the cache dequantized
before (or inside) attention, with the arithmetic itself done in high
precision.

Readings: query head h reads KV head h // n_rep
(contiguous blocks of query heads share a KV head); the scale is
1/sqrt(head_dim); one decode query per sequence attends to every cached
token (sinks, quantized body, fp16 residual) with no mask; the softmax
subtracts the row maximum before exponentiating.
"""
from __future__ import annotations

import math

import numpy as np


def attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray) -> np.ndarray:
    """out[b, h] = sum_t softmax_t(q[b,h] . k_hat[b, h//n_rep, t] / sqrt(D)) v_hat[...].

    q: [B][Hq][D] (any float dtype, upcast exactly); k_hat, v_hat:
    [B][Hkv][n][D] fp64.  Returns [B][Hq][D] fp64.
    """
    q = np.asarray(q).astype(np.float64)
    b, hq, d = q.shape
    hkv = k_hat.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    n_rep = hq // hkv
    qg = q.reshape(b, hkv, n_rep, d)
    logits = np.einsum("bgrd,bgtd->bgrt", qg, k_hat) / math.sqrt(d)
    logits -= logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=-1, keepdims=True)
    out = np.einsum("bgrt,bgtd->bgrd", p, v_hat)
    return out.reshape(b, hq, d)


def attention_loops(q, k_hat, v_hat) -> np.ndarray:
    """The same quantity with explicit Python loops (for tiny inputs only)."""
    q = np.asarray(q).astype(np.float64)
    b, hq, d = q.shape
    hkv, n = k_hat.shape[1], k_hat.shape[2]
    n_rep = hq // hkv
    out = np.zeros((b, hq, d))
    for bi in range(b):
        for h in range(hq):
            g = h // n_rep
            ell = []
            for t in range(n):
                acc = 0.0
                for c in range(d):
                    acc += q[bi, h, c] * k_hat[bi, g, t, c]
                ell.append(acc / math.sqrt(d))
            m = max(ell)
            w = [math.exp(x - m) for x in ell]
            tot = math.fsum(w)
            for c in range(d):
                out[bi, h, c] = math.fsum(w[t] * v_hat[bi, g, t, c] for t in range(n)) / tot
    return out
