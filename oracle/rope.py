"""Rotary position embedding of the Keys, for caches that store Keys before RoPE.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"KV Cache Quantization Analysis", sec. 3 (RoPE problem) and sec. 4
(KVQuant): the rotary position encoding mixes channel pairs and spreads the
Key outlier channels, so KVQuant quantizes the Keys per channel *before*
RoPE; the rotation is then applied to the dequantized Keys.

The pages do not write the rotation out.  Readings:

* the rotate-half convention of the Llama family: channel i and channel
  i + D/2 (i < D/2) form a pair rotated by the angle pos * theta_i, with
  theta_i = base^(-2i/D) and a configurable base ("rope theta");
* pos is the token's index in the sequence (0-based, sinks included);
* the decode query arrives already rotated at its own position, so only the
  Keys are rotated here; the logit then depends on positions only through
  their difference;
* the angles, cosines and sines are fp64.
"""
from __future__ import annotations

import numpy as np


def frequencies(d: int, theta: float) -> np.ndarray:
    """theta_i = theta^(-2i/d) for i < d/2, fp64."""
    if d % 2:
        raise ValueError("head_dim must be even")
    return np.float64(theta) ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)


def apply_rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate rows of x [..., n, D] at positions pos [n] (rotate-half pairs), fp64."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, np.float64)[:, None] * frequencies(d, theta)[None, :]    # [n, D/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def stored_channel(p: np.ndarray, d: int) -> np.ndarray:
    """Channel held by stored position p of a pre-RoPE Key row: pairs side by side,
    position 2i -> channel i, position 2i + 1 -> channel i + d/2."""
    p = np.asarray(p)
    return (p >> 1) + (d // 2) * (p & 1)
