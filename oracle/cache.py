"""Token routing of the quantized KV cache, stated as a pure function of history.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix
------------------
* "KV Cache Quantization Analysis", sec. 5 (system integration): the new
  token's K and V are quantized right after they are computed and stored;
  they are dequantized just before attention.
* Same page, sec. 3 and sec. 4 (KIVI): the most recent tokens are kept in
  full precision as a sliding window (the "residual"); Keys are quantized
  per channel, Values per token.
* "W4A16 + KV cache quantization: combined accuracy", section on layer
  sensitivity: keeping the attention-sink tokens' K/V in FP16 recovers most
  of the quality.

Readings where the pages are silent:

* The first ``S`` absolute tokens are sinks, stored verbatim (fp16).
* The other tokens form the body, indexed u = t - S.  Per-channel Keys need
  a whole group of G tokens before a group can be quantized, so the window
  is "at least R tokens, flushed G at a time": after n tokens,
  n_q = G * floor(max(0, n_body - R) / G) body tokens are quantized and the
  remaining r = n_body - n_q (R <= r < R + G once n_body >= R) stay fp16.
* K and V share the one boundary n_q.  FP8 uses the same G-token blocks
  (no metadata), so every format has the same window.
* A residual body token u lives in ring slot u mod (R + G).
* Every sequence of the batch holds the same number of tokens.

Because each group is quantized once, from the original fp16 values, and
never re-quantized, the cache after any sequence of appends is a function of
the token history only.  :func:`build_cache` computes it that way; the GPU
library appends incrementally and must land on the same state for every
chunking of the same history.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import quant

FORMATS = ("int8", "int4", "int2", "fp8", "fp8_e5m2")
FP8_FORMATS = ("fp8", "fp8_e5m2")
BITS = {"int8": 8, "int4": 4, "int2": 2, "fp8": 8, "fp8_e5m2": 8}


@dataclass
class Layout:
    """Logical description of one layer's cache (mirrors the C layout struct)."""
    batch: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    max_tokens: int
    fmt: str
    k_group_tokens: int = 32
    v_group_channels: int = 32
    residual_tokens: int = 128
    sink_tokens: int = 0
    k_scale: float = 1.0
    v_scale: float = 1.0
    meta_fp16: bool = False       # INT only: fp16 (s, m) pairs instead of fp32 (s, z)
    rope_theta: float = 0.0       # > 0: Keys stored before RoPE, rotated with this base in attention
    outliers: bool = False        # INT only: one exact fp16 outlier per quantization group

    @property
    def bits(self) -> int:
        return BITS[self.fmt]

    @property
    def n_rep(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def ring_slots(self) -> int:
        return self.residual_tokens + self.k_group_tokens


def window_split(n: int, sink: int, residual: int, group: int):
    """(n_sink, n_q, r) after n tokens: sinks kept, body tokens quantized, residual."""
    n_sink = min(n, sink)
    n_body = max(0, n - sink)
    n_q = group * (max(0, n_body - residual) // group)
    return n_sink, n_q, n_body - n_q


@dataclass
class CacheState:
    """Logical contents of a cache after n tokens (all arrays numpy)."""
    layout: Layout
    n: int
    n_sink: int
    n_q: int
    r: int
    sink_k: np.ndarray            # [B][Hkv][n_sink][D] fp16
    sink_v: np.ndarray
    codes_k: np.ndarray           # [B][Hkv][n_q][D] uint8 (int codes or E4M3 bytes)
    codes_v: np.ndarray
    s_k: np.ndarray | None        # [B][Hkv][n_q/G_k][D] fp32 (INT only; fp16 with meta_fp16)
    z_k: np.ndarray | None        # zero-point z (fp32), or the fp16 offset m with meta_fp16
    s_v: np.ndarray | None        # [B][Hkv][n_q][D/G_v], as s_k / z_k
    z_v: np.ndarray | None
    res_k: np.ndarray             # [B][Hkv][r][D] fp16, body order
    res_v: np.ndarray
    res_slots: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    # outliers: K [B][Hkv][n_q/G_k][D] token index in the block and fp16 value;
    # V [B][Hkv][n_q][D/G_v] channel index in the group and fp16 value
    ko_idx: np.ndarray | None = None
    ko_val: np.ndarray | None = None
    vo_idx: np.ndarray | None = None
    vo_val: np.ndarray | None = None


def build_cache(k: np.ndarray, v: np.ndarray, lay: Layout) -> CacheState:
    """State of the cache after appending the token history ``k``, ``v``.

    ``k`` and ``v`` are fp16 arrays [B][n][Hkv][D] (all tokens ever appended,
    in order).  Groups are quantized independently from the fp16 values.
    """
    k = np.asarray(k, np.float16)
    v = np.asarray(v, np.float16)
    b, n, hkv, d = k.shape
    assert v.shape == k.shape
    g = lay.k_group_tokens
    n_sink, n_q, r = window_split(n, lay.sink_tokens, lay.residual_tokens, g)
    kt = np.transpose(k, (0, 2, 1, 3))           # [B][Hkv][n][D]
    vt = np.transpose(v, (0, 2, 1, 3))
    s0 = lay.sink_tokens
    body_k = kt[:, :, n_sink:n_sink + n_q]       # body tokens u < n_q (sinks come first)
    body_v = vt[:, :, n_sink:n_sink + n_q]
    s_k = z_k = s_v = z_v = None
    if lay.fmt in FP8_FORMATS:
        codes_k = quant.fp8_encode(body_k, lay.k_scale, lay.fmt)
        codes_v = quant.fp8_encode(body_v, lay.v_scale, lay.fmt)
    else:
        bits = lay.bits
        kg = body_k.reshape(b, hkv, n_q // g, g, d)
        if lay.outliers:
            ck, s_k, z_k, ko_i, ko_v = quant.quantize_k_group(kg, bits, lay.meta_fp16, outliers=True)
            codes_v, s_v, z_v, vo_i, vo_v = quant.quantize_v_tokens(body_v, bits, lay.v_group_channels,
                                                                    lay.meta_fp16, outliers=True)
        else:
            ck, s_k, z_k = quant.quantize_k_group(kg, bits, lay.meta_fp16)
            codes_v, s_v, z_v = quant.quantize_v_tokens(body_v, bits, lay.v_group_channels, lay.meta_fp16)
        codes_k = ck.reshape(b, hkv, n_q, d)
    res_k = kt[:, :, s0 + n_q:]
    res_v = vt[:, :, s0 + n_q:]
    assert res_k.shape[2] == r
    slots = (np.arange(n_q, n_q + r) % lay.ring_slots).astype(np.int64)
    st = CacheState(lay, n, n_sink, n_q, r, kt[:, :, :n_sink].copy(), vt[:, :, :n_sink].copy(),
                    codes_k, codes_v, s_k, z_k, s_v, z_v, res_k.copy(), res_v.copy(), slots)
    if lay.fmt not in FP8_FORMATS and lay.outliers:
        st.ko_idx, st.ko_val, st.vo_idx, st.vo_val = ko_i, ko_v, vo_i, vo_v
    return st


def dequantize(st: CacheState):
    """(K_hat, V_hat) in fp64, [B][Hkv][n][D], in absolute token order.

    For a pre-RoPE cache (rope_theta > 0) K_hat is the dequantized Key before
    the rotation; :func:`attention_keys` applies it.
    """
    lay = st.layout
    if lay.fmt in FP8_FORMATS:
        kq = quant.fp8_decode(st.codes_k, lay.k_scale, lay.fmt)
        vq = quant.fp8_decode(st.codes_v, lay.v_scale, lay.fmt)
    else:
        b, hkv, n_q, d = st.codes_k.shape
        g = lay.k_group_tokens
        kq = quant.dequantize_k_group(st.codes_k.reshape(b, hkv, n_q // g, g, d),
                                      st.s_k, st.z_k, st.ko_idx, st.ko_val).reshape(b, hkv, n_q, d)
        vq = quant.dequantize_v_tokens(st.codes_v, st.s_v, st.z_v, st.vo_idx, st.vo_val)
    kh = np.concatenate([st.sink_k.astype(np.float64), kq, st.res_k.astype(np.float64)], axis=2)
    vh = np.concatenate([st.sink_v.astype(np.float64), vq, st.res_v.astype(np.float64)], axis=2)
    return kh, vh


def attention_keys(st: CacheState, k_hat: np.ndarray) -> np.ndarray:
    """The Keys attention uses: K_hat itself, or for a pre-RoPE cache K_hat
    rotated at each token's position t = 0 .. n-1 ("KV Cache Quantization
    Analysis", sec. 4, KVQuant: quantize before RoPE, rotate after)."""
    if not st.layout.rope_theta:
        return k_hat
    from .rope import apply_rope
    return apply_rope(k_hat, np.arange(k_hat.shape[-2]), st.layout.rope_theta)
