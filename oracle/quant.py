"""Quantization codecs of the KV cache, written out in numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Integer formats (INT8 / INT4 / INT2)
------------------------------------
"KV Cache Quantization Analysis", sec. 2 (quantization basics) gives uniform
affine quantization: a real x maps to the integer q = round(x/s + z) and back
to x_hat = s * (q - z), with s the scale and z the zero-point; an asymmetric
z (non-zero) is preferred when the data is not centred on zero; per-channel /
per-token granularity stores one (s, z) pair per row or column.

Readings taken where the page is silent:

* range estimator: s and z map the group minimum to code 0 and the group
  maximum to code 2^b - 1 (plain min/max, no clipping);
* every step is one IEEE fp32 operation with round-to-nearest-even, in the
  order the formula is written: s = (max - min) / (2^b - 1), z = (-min) / s,
  q = clamp(rint(x / s + z), 0, 2^b - 1); true division, no fused
  multiply-add;
* z is kept real-valued (fp32), not rounded to an integer;
* a constant group (max == min) gets s = 1, so every code is 0 and the
  dequantized value equals the constant exactly;
* the group minimum is normalised with ``+ 0.0`` so that a zero minimum is
  always +0 (then z is -0.0, bit pattern 0x80000000);
* dequantization x_hat = s * (q - z) is evaluated in fp64 from the stored
  fp32 s and z.

FP8 E4M3
--------
Sec. 4 of the same page (FP8 / INT8) names the OCP E4M3 format (4 exponent
bits, 3 mantissa bits) used with an fp32 scale.  The page prints a +-240
range, which is the maximum of the "fnuz" E4M3 variant; the OCP format the
page names has maximum finite magnitude 448 (exponent bias 7, no infinities,
S.1111.111 is NaN).  This oracle uses OCP E4M3 with max 448 and restates the
codec from the format definition: the encoder rounds to nearest, ties to the
even code, after an explicit clamp to [-448, 448]; the sign of zero is kept.
The scale is symmetric and per tensor: v = x / s in fp32, code = E4M3(v),
x_hat = s * decode(code).

FP8 E5M2
--------
The same section names OCP E5M2 (5 exponent bits, 2 mantissa bits) as the
other FP8 format.  OCP E5M2: exponent bias 15, subnormals 2^-14 * M/4,
exponent 31 holds the infinities (M = 0) and NaNs (M != 0), largest finite
magnitude 57344.  It is used exactly like E4M3: explicit clamp of x / s to
[-57344, 57344], round to nearest with ties to the even code, one fp32 scale
per tensor.

fp16 scale / offset metadata (INT formats)
------------------------------------------
The 27B KL-divergence study's table of KV-cache sizes per token (34 : 32 : 18
KiB for 8-bit block formats, FP8 and 4-bit block formats) works out to one
16-bit scale per 32 values.  The fp16-metadata variant stores 16 bits per
scale and per offset.  Readings:

* an fp16 zero-point z = -min / s would lose the s/2 error bound whenever
  |z| is large (its rounding error is up to |z| * 2^-11 code steps), so the
  offset is stored in value units instead: m = min, which an fp16 group
  holds exactly.  The affine map is the same, x_hat = s * (q - z) with
  s * z = -m;
* s is (max - min) / (2^b - 1) in fp32, then rounded *up* to the nearest
  fp16 (the smallest fp16 >= the fp32 value), so the group's range still
  fits the codes; a constant group gets s = 1;
* q = clamp(rint((x - m) / s), 0, 2^b - 1), each step one fp32 operation
  (subtraction, true division, rint) on the stored fp16 s and m;
* x_hat = s * q + m, in fp64 from the stored fp16 values.

Dense-and-sparse outliers (INT formats)
---------------------------------------
"KV Cache Quantization Analysis", sec. 2 (outliers: a few large values widen
the grid and cost every other value resolution) and sec. 4 (KVQuant, its
fourth component: per-vector dense-and-sparse quantization keeps outliers
apart from the quantized values).  The pages give no outlier count or
selection rule.  Readings:

* one outlier per quantization group (the vector: a Key channel's 32 tokens
  of a block, a Value token's 32-channel group), about 3 % of the values;
* the outlier is the value of largest magnitude, the lowest index on ties;
* it is stored exactly (fp16) with its index; the group's scale and
  zero-point (or fp16 scale and offset) come from the other 31 values with
  the formulas above; its own code is 0;
* x_hat is the stored outlier at its index and the affine decode elsewhere.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# --------------------------------------------------------------------------
# Integer affine quantization
# --------------------------------------------------------------------------


def int_qmax(bits: int) -> int:
    """Largest code of a b-bit unsigned code (2^b - 1)."""
    if bits not in (2, 4, 8):
        raise ValueError(f"unsupported bit width {bits}")
    return (1 << bits) - 1


def int_group_params(x: np.ndarray, bits: int, axis):
    """Scale and zero-point of each group of ``x`` reduced over ``axis``.

    ``x`` must be float32 (exact upcast of the fp16 cache input).  Returns
    (s, z) as float32 arrays with ``axis`` removed.  Follows the affine
    formula of "KV Cache Quantization Analysis", sec. 2, with the min/max
    range reading stated in the module docstring.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("int_group_params expects float32 input")
    qmax = F32(int_qmax(bits))
    mn = x.min(axis=axis) + F32(0.0)          # -0 -> +0
    mx = x.max(axis=axis)
    s = (mx - mn) / qmax                       # fp32 true division, RNE
    s = np.where(s == F32(0.0), F32(1.0), s).astype(F32)
    z = (-mn) / s                              # fp32, real-valued zero-point
    return s.astype(F32), z.astype(F32)


def int_encode(x: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int) -> np.ndarray:
    """q = clamp(rint(x / s + z), 0, 2^b - 1) in fp32 steps; returns uint8.

    ``s`` and ``z`` must broadcast against ``x``.
    """
    x = np.asarray(x, dtype=F32)
    s = np.asarray(s, dtype=F32)
    z = np.asarray(z, dtype=F32)
    v = (x / s) + z                            # two separately rounded fp32 ops
    q = np.rint(v)                             # round half to even
    q = np.clip(q, F32(0.0), F32(int_qmax(bits)))
    return q.astype(np.uint8)


def int_decode(q: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """x_hat = s * (q - z), evaluated in fp64 from the stored fp32 s, z."""
    return np.asarray(s, np.float64) * (np.asarray(q, np.float64) - np.asarray(z, np.float64))


def f16_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest fp16 value >= x (x finite, >= 0, at most 65504)."""
    x = np.asarray(x, F32)
    h = x.astype(np.float16)                               # round to nearest even
    low = h.astype(F32) < x
    with np.errstate(over="ignore"):                       # 65504 steps to inf where unused
        up = np.nextafter(h, np.float16(np.inf))
    return np.where(low, up, h).astype(np.float16)


def int_group_params_f16(x: np.ndarray, bits: int, axis):
    """fp16 scale and offset of each group of ``x`` reduced over ``axis``.

    ``x`` is float32 holding fp16 values.  Returns (s, m) as float16 arrays:
    s = (max - min) / (2^b - 1) in fp32 rounded up to fp16 (1 for a constant
    group) and m = min (exact in fp16).
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("int_group_params_f16 expects float32 input")
    qmax = F32(int_qmax(bits))
    mn = x.min(axis=axis) + F32(0.0)          # -0 -> +0
    mx = x.max(axis=axis)
    s = f16_round_up((mx - mn) / qmax)
    s = np.where(s == np.float16(0.0), np.float16(1.0), s).astype(np.float16)
    m = mn.astype(np.float16)
    assert np.array_equal(m.astype(F32), mn), "group minimum must be an fp16 value"
    return s, m


def int_encode_offset(x: np.ndarray, s: np.ndarray, m: np.ndarray, bits: int) -> np.ndarray:
    """q = clamp(rint((x - m) / s), 0, 2^b - 1) in fp32 steps; returns uint8."""
    x = np.asarray(x, dtype=F32)
    s = np.asarray(s, dtype=np.float16).astype(F32)
    m = np.asarray(m, dtype=np.float16).astype(F32)
    v = (x - m) / s                            # two separately rounded fp32 ops
    q = np.rint(v)
    q = np.clip(q, F32(0.0), F32(int_qmax(bits)))
    return q.astype(np.uint8)


def int_decode_offset(q: np.ndarray, s: np.ndarray, m: np.ndarray) -> np.ndarray:
    """x_hat = s * q + m, in fp64 from the stored fp16 s, m."""
    return np.asarray(s, np.float64) * np.asarray(q, np.float64) + np.asarray(m, np.float64)


def outlier_index(x: np.ndarray, axis: int) -> np.ndarray:
    """Index along ``axis`` of each group's value of largest magnitude (lowest index on ties)."""
    a = np.abs(np.moveaxis(np.asarray(x, F32), axis, -1))
    n = a.shape[-1]
    # sort key: larger magnitude first, then smaller index
    order = np.lexsort((np.broadcast_to(np.arange(n), a.shape), -a), axis=-1)
    return order[..., 0]


def _dense_params(x: np.ndarray, bits: int, axis: int, meta16: bool):
    """Group parameters over all values except each group's outlier."""
    xm = np.moveaxis(np.asarray(x, F32), axis, -1)
    idx = outlier_index(xm, -1)
    keep = np.ones(xm.shape, bool)
    np.put_along_axis(keep, idx[..., None], False, axis=-1)
    # the excluded value is replaced by a value already in the group (its
    # neighbour), which leaves min and max of the others unchanged
    nb = np.take_along_axis(xm, np.where(idx == 0, 1, 0)[..., None], axis=-1)
    xd = np.where(keep, xm, nb)
    params = int_group_params_f16(xd, bits, -1) if meta16 else int_group_params(xd, bits, -1)
    val = np.take_along_axis(xm, idx[..., None], axis=-1)[..., 0].astype(np.float16)
    return params, idx, val


def quantize_k_group(kg: np.ndarray, bits: int, meta16: bool = False, outliers: bool = False):
    """Key group of shape [..., G_k tokens, D]: per-channel (s, z) over tokens.

    "KV Cache Quantization Analysis", sec. 3: a few fixed Key channels hold
    large values, so each channel gets its own scale (per-channel Keys).
    Returns codes [..., G_k, D] uint8 and s, z [..., D] float32 (with
    ``meta16``: fp16 scale s and fp16 offset m in place of z).
    """
    x = np.asarray(kg, np.float16).astype(F32)
    if outliers:
        (s, z), idx, val = _dense_params(x, bits, -2, meta16)
        enc = int_encode_offset if meta16 else int_encode
        q = enc(x, s[..., None, :], z[..., None, :], bits)
        np.put_along_axis(q, idx[..., None, :], 0, axis=-2)
        return q, s, z, idx, val
    if meta16:
        s, m = int_group_params_f16(x, bits, axis=-2)
        return int_encode_offset(x, s[..., None, :], m[..., None, :], bits), s, m
    s, z = int_group_params(x, bits, axis=-2)
    q = int_encode(x, s[..., None, :], z[..., None, :], bits)
    return q, s, z


def quantize_v_tokens(v: np.ndarray, bits: int, g_v: int, meta16: bool = False, outliers: bool = False):
    """Values of shape [..., T, D]: per-token (s, z) over groups of g_v channels.

    "KV Cache Quantization Analysis", sec. 3: the attention output mixes
    Value rows, so errors are confined per token (per-token Values).
    Returns codes [..., T, D] uint8 and s, z [..., T, D // g_v] float32 (with
    ``meta16``: fp16 s and offset m).
    """
    x = np.asarray(v, np.float16).astype(F32)
    d = x.shape[-1]
    if d % g_v:
        raise ValueError("head_dim must be a multiple of the V channel group")
    xg = x.reshape(x.shape[:-1] + (d // g_v, g_v))
    if outliers:
        (s, z), idx, val = _dense_params(xg, bits, -1, meta16)
        enc = int_encode_offset if meta16 else int_encode
        q = enc(xg, s[..., None], z[..., None], bits)
        np.put_along_axis(q, idx[..., None], 0, axis=-1)
        return q.reshape(x.shape), s, z, idx, val
    if meta16:
        s, m = int_group_params_f16(xg, bits, axis=-1)
        return int_encode_offset(xg, s[..., None], m[..., None], bits).reshape(x.shape), s, m
    s, z = int_group_params(xg, bits, axis=-1)
    q = int_encode(xg, s[..., None], z[..., None], bits)
    return q.reshape(x.shape), s, z


def _decode(q, s, z):
    """fp32 (s, z) pairs decode as s * (q - z); fp16 (s, m) pairs as s * q + m."""
    if np.asarray(s).dtype == np.float16:
        return int_decode_offset(q, s, z)
    return int_decode(q, s, z)


def dequantize_k_group(q: np.ndarray, s: np.ndarray, z: np.ndarray, idx=None, val=None) -> np.ndarray:
    """Inverse of :func:`quantize_k_group` in fp64 (outliers, if given, restored exactly)."""
    x = _decode(q, s[..., None, :], z[..., None, :])
    if idx is not None:
        np.put_along_axis(x, np.asarray(idx)[..., None, :], np.asarray(val, np.float64)[..., None, :], axis=-2)
    return x


def dequantize_v_tokens(q: np.ndarray, s: np.ndarray, z: np.ndarray, idx=None, val=None) -> np.ndarray:
    """Inverse of :func:`quantize_v_tokens` in fp64 (outliers, if given, restored exactly)."""
    d = q.shape[-1]
    g = s.shape[-1]
    qg = q.reshape(q.shape[:-1] + (g, d // g))
    x = _decode(qg, s[..., None], z[..., None])
    if idx is not None:
        np.put_along_axis(x, np.asarray(idx)[..., None], np.asarray(val, np.float64)[..., None], axis=-1)
    return x.reshape(q.shape)


# --------------------------------------------------------------------------
# OCP FP8 E4M3
# --------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def e4m3_decode_table() -> np.ndarray:
    """Value of every one of the 256 E4M3 codes (fp64; NaN for 0x7F/0xFF).

    Bit layout S EEEE MMM, exponent bias 7.  E == 0 is subnormal:
    (-1)^S * 2^-6 * M/8; otherwise (-1)^S * 2^(E-7) * (1 + M/8).  E == 15 with
    M == 7 is NaN; there are no infinities.
    """
    out = np.empty(256, np.float64)
    for c in range(256):
        sgn = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sgn * (2.0 ** -6) * (m / 8.0)
        else:
            out[c] = sgn * (2.0 ** (e - 7)) * (1.0 + m / 8.0)
    return out


_E4M3 = e4m3_decode_table()
_E4M3_POS = _E4M3[:0x7F]          # codes 0x00..0x7E, strictly increasing, 0 .. 448


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round finite values with |v| <= 448 to the nearest E4M3 code.

    Ties go to the code with an even mantissa (even code).  The sign bit is
    taken from the input, so -0.0 encodes to 0x80.  Values outside
    [-448, 448] raise: callers clamp first.
    """
    v = np.asarray(v, np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode needs finite values within +-448")
    a = np.abs(v)
    hi = np.searchsorted(_E4M3_POS, a, side="left")       # table[hi-1] < a <= table[hi]
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]                                 # exact in fp64
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3_POS[hi], hi, code).astype(np.uint8)
    neg = np.signbit(v)
    return (code | np.where(neg, 0x80, 0x00)).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """E4M3 code -> value (fp64)."""
    return _E4M3[np.asarray(code, np.uint8)]


E5M2_MAX = 57344.0


def e5m2_decode_table() -> np.ndarray:
    """Value of every one of the 256 E5M2 codes (fp64; +-inf, NaN included).

    Bit layout S EEEEE MM, exponent bias 15.  E == 0 is subnormal:
    (-1)^S * 2^-14 * M/4; E == 31 is +-infinity (M == 0) or NaN (M != 0);
    otherwise (-1)^S * 2^(E-15) * (1 + M/4).
    """
    out = np.empty(256, np.float64)
    for c in range(256):
        sgn = -1.0 if c & 0x80 else 1.0
        e = (c >> 2) & 0x1F
        m = c & 0x3
        if e == 0x1F:
            out[c] = sgn * np.inf if m == 0 else np.nan
        elif e == 0:
            out[c] = sgn * (2.0 ** -14) * (m / 4.0)
        else:
            out[c] = sgn * (2.0 ** (e - 15)) * (1.0 + m / 4.0)
    return out


_E5M2 = e5m2_decode_table()
_E5M2_POS = _E5M2[:0x7C]          # codes 0x00..0x7B, strictly increasing, 0 .. 57344


def _nearest_code(v: np.ndarray, pos: np.ndarray, vmax: float, name: str) -> np.ndarray:
    """Nearest code of a strictly increasing table of non-negative values.

    Ties go to the even code; the sign bit comes from the input.
    """
    v = np.asarray(v, np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > vmax):
        raise ValueError(f"{name} needs finite values within +-{vmax:g}")
    a = np.abs(v)
    hi = np.searchsorted(pos, a, side="left")              # pos[hi-1] < a <= pos[hi]
    hi = np.minimum(hi, len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - pos[lo]                                       # exact in fp64
    dhi = pos[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == pos[hi], hi, code).astype(np.uint8)
    neg = np.signbit(v)
    return (code | np.where(neg, 0x80, 0x00)).astype(np.uint8)


def e5m2_encode(v: np.ndarray) -> np.ndarray:
    """Round finite values with |v| <= 57344 to the nearest E5M2 code (ties even)."""
    return _nearest_code(v, _E5M2_POS, E5M2_MAX, "e5m2_encode")


def e5m2_decode(code: np.ndarray) -> np.ndarray:
    """E5M2 code -> value (fp64)."""
    return _E5M2[np.asarray(code, np.uint8)]


FP8_MAX = {"fp8": E4M3_MAX, "fp8_e5m2": E5M2_MAX}


def fp8_scale(x_prefill: np.ndarray, fmt: str = "fp8") -> np.float32:
    """Per-tensor scale used by the tests: amax(|x|) / max (1 if all 0).

    Sec. 5 of the analysis page says calibrated scales improve FP8 quality;
    the scale is a fixed input of the cache once set.  This recipe is the
    plainest calibration: map the largest magnitude seen at prefill to the
    format's largest finite value (448 for E4M3, 57344 for E5M2).
    """
    a = F32(np.max(np.abs(np.asarray(x_prefill, np.float16).astype(F32))))
    if a == F32(0.0):
        return F32(1.0)
    return F32(a / F32(FP8_MAX[fmt]))


def fp8_encode(x: np.ndarray, s, fmt: str = "fp8") -> np.ndarray:
    """code = FP8_RNE(clamp(x / s, -max, max)), with x / s one fp32 division."""
    vmax = FP8_MAX[fmt]
    v = np.asarray(x, np.float16).astype(F32) / F32(s)
    v = np.clip(v, F32(-vmax), F32(vmax))
    return e4m3_encode(v) if fmt == "fp8" else e5m2_encode(v)


def fp8_decode(code: np.ndarray, s, fmt: str = "fp8") -> np.ndarray:
    """x_hat = s * decode(code) in fp64."""
    dec = e4m3_decode(code) if fmt == "fp8" else e5m2_decode(code)
    return np.float64(F32(s)) * dec
