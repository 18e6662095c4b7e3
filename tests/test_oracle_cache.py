"""Pins of the oracle's routing, attention and byte counter."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, cache, layout, nbytes, quant
from quantized_kv_cache_quant_amd import synth


def _lay(fmt="int4", b=1, hkv=1, hq=4, d=128, n=256, r=32, s=0, **kw):
    return cache.Layout(b, hkv, hq, d, n + 64, fmt, residual_tokens=r, sink_tokens=s, **kw)


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("name,n_q,r", [("tiny", 224, 32), ("llama3_8b", 8064, 128),
                                        ("llama3_8b_kivi2", 8064, 128), ("llama3_70b", 8032, 156),
                                        ("long_ctx", 130944, 128)])
def test_window_split_of_the_workloads(name, n_q, r):
    w = synth.WORKLOADS[name]
    ns, nq, rr = cache.window_split(w.seq_len, w.sink_tokens, w.residual_tokens, w.k_group_tokens)
    assert (ns, nq, rr) == (w.sink_tokens, n_q, r)


def test_window_invariants():
    for n in range(0, 400):
        for s in (0, 4):
            for r in (0, 1, 32, 128):
                ns, nq, rr = cache.window_split(n, s, r, 32)
                assert ns + nq + rr == n and nq % 32 == 0
                if n - ns >= r:
                    assert r <= rr < r + 32
                else:
                    assert nq == 0


class _RingSim:
    """Independent token-by-token simulation: fp16 ring of R+G slots, flush G at a time."""

    def __init__(self, lay):
        self.lay = lay
        self.ring_k = {}
        self.sinks = []
        self.groups = []          # list of K groups [G][Hkv][D] as they are flushed
        self.n = 0
        self.nq = 0

    def push(self, k_tok):
        lay = self.lay
        if self.n < lay.sink_tokens:
            self.sinks.append(k_tok)
        else:
            u = self.n - lay.sink_tokens
            self.ring_k[u % lay.ring_slots] = (u, k_tok)
            while (u + 1) - self.nq >= lay.residual_tokens + lay.k_group_tokens:
                grp = []
                for uu in range(self.nq, self.nq + lay.k_group_tokens):
                    slot_u, tok = self.ring_k[uu % lay.ring_slots]
                    assert slot_u == uu                     # never overwritten before flush
                    grp.append(tok)
                self.groups.append(np.stack(grp))
                self.nq += lay.k_group_tokens
        self.n += 1


@pytest.mark.parametrize("s,r", [(0, 32), (4, 32), (0, 0), (3, 5)])
def test_build_cache_equals_incremental_ring(s, r):
    lay = _lay("int4", b=1, hkv=2, hq=4, d=32, n=300, r=r, s=s)
    k, v = synth.kv_tokens(synth.WORKLOADS["tiny"], 11, 12, 1, 300, 2, 32)
    sim = _RingSim(lay)
    for t in range(300):
        sim.push(k[0, t])
        st = cache.build_cache(k[:, :t + 1], v[:, :t + 1], lay)
        assert st.n_q == sim.nq and st.n_sink == len(sim.sinks)
        for j, grp in enumerate(sim.groups):               # groups from the ring = from history
            ref, _, _ = quant.quantize_k_group(np.transpose(grp, (1, 0, 2)), 4)
            assert np.array_equal(st.codes_k[0, :, j * 32:(j + 1) * 32], ref)
        for i, slot in enumerate(st.res_slots):             # residual tokens sit in their slots
            uu, tok = sim.ring_k[slot]
            assert uu == st.n_q + i
            assert np.array_equal(st.res_k[0, :, i], tok)


# ---------------------------------------------------------------- attention
def test_attention_loops_equal_vectorized():
    w = synth.WORKLOADS["tiny"]
    lay = _lay("int4", d=16, n=70, r=8, v_group_channels=8)
    k, v = synth.kv_tokens(w, 1, 2, 1, 70, 1, 16)
    q = synth.queries(w, 1, 4, 16)
    kh, vh = cache.dequantize(cache.build_cache(k, v, lay))
    a = attention.attention(q, kh, vh)
    b = attention.attention_loops(q, kh, vh)
    assert np.max(np.abs(a - b)) < 1e-12


def test_attention_equals_sdpa_when_nothing_is_quantized():
    w = synth.WORKLOADS["llama3_8b"]
    b, hq, hkv, d, n = 2, 8, 2, 64, 100
    lay = cache.Layout(b, hkv, hq, d, n, "int8", residual_tokens=n)
    k, v = synth.kv_tokens(w, 5, 6, b, n, hkv, d)
    q = synth.queries(w, b, hq, d)
    st = cache.build_cache(k, v, lay)
    assert st.n_q == 0
    kh, vh = cache.dequantize(st)
    ours = attention.attention(q, kh, vh)
    kt = torch.from_numpy(kh).repeat_interleave(hq // hkv, dim=1)
    vt = torch.from_numpy(vh).repeat_interleave(hq // hkv, dim=1)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0].numpy()
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_attention_closed_forms():
    rng = np.random.default_rng(0)
    b, hkv, n, d = 1, 2, 50, 32
    kh = rng.standard_normal((b, hkv, n, d))
    vv = rng.standard_normal((b, hkv, 1, d))
    q = rng.standard_normal((b, 4, d))
    out = attention.attention(q, kh, np.repeat(vv, n, axis=2))   # all V rows equal
    assert np.max(np.abs(out - np.repeat(vv[:, :, 0], 2, axis=1))) < 1e-12
    vh = rng.standard_normal((b, hkv, n, d))
    out = attention.attention(np.zeros((b, 4, d)), kh, vh)          # q = 0 -> mean of V
    assert np.max(np.abs(out - np.repeat(vh.mean(axis=2), 2, axis=1))) < 1e-12
    k2 = np.zeros((b, hkv, n, d)); k2[:, :, 17, 0] = 50.0 * math.sqrt(d) * 4
    q2 = np.zeros((b, 4, d)); q2[:, :, 0] = 1.0                      # token 17 dominates
    out = attention.attention(q2, k2, vh)
    assert np.max(np.abs(out - np.repeat(vh[:, :, 17], 2, axis=1))) < 1e-12


def test_attention_permutation_and_mha():
    rng = np.random.default_rng(1)
    kh = rng.standard_normal((2, 3, 40, 16)); vh = rng.standard_normal((2, 3, 40, 16))
    q = rng.standard_normal((2, 6, 16))
    p = rng.permutation(40)
    a = attention.attention(q, kh, vh)
    assert np.max(np.abs(a - attention.attention(q, kh[:, :, p], vh[:, :, p]))) < 1e-12
    # n_rep = 1 is multi-head attention: head h reads KV head h
    q1 = rng.standard_normal((2, 3, 16))
    m = attention.attention(q1, kh, vh)
    for h in range(3):
        single = attention.attention(q1[:, h:h + 1], kh[:, h:h + 1], vh[:, h:h + 1])
        assert np.max(np.abs(m[:, h] - single[:, 0])) < 1e-12
    # contiguous GQA blocks: heads 0,1 share KV head 0
    assert np.max(np.abs(a[:, 0] - attention.attention(q[:, 0:1], kh[:, :1], vh[:, :1])[:, 0])) < 1e-12
    assert np.max(np.abs(a[:, 3] - attention.attention(q[:, 3:4], kh[:, 1:2], vh[:, 1:2])[:, 0])) < 1e-12


# -------------------------------------------------- qualitative sanity gates
def _attn_err(st, q, k, v):
    kh, vh = cache.dequantize(st)
    kt = np.transpose(k, (0, 2, 1, 3)).astype(np.float64)
    vt = np.transpose(v, (0, 2, 1, 3)).astype(np.float64)
    return np.mean(np.abs(attention.attention(q, kh, vh) - attention.attention(q, kt, vt)))


def test_per_channel_keys_beat_per_token_keys_with_outliers():
    w = synth.WORKLOADS["tiny"]
    k, _ = synth.kv_tokens(w, 1001, 2001, 1, 256)
    x = np.transpose(k, (0, 2, 1, 3))[0, 0].astype(np.float32)      # [256][128]
    xg = x.reshape(8, 32, 128)
    qc, sc, zc = quant.quantize_k_group(xg, 4)                      # per channel
    e_ch = np.abs(quant.dequantize_k_group(qc, sc, zc).reshape(256, 128) - x).mean()
    qt, st_, zt = quant.quantize_v_tokens(x, 4, 128)                 # per token (whole row)
    e_tok = np.abs(quant.dequantize_v_tokens(qt, st_, zt) - x).mean()
    assert e_ch < 0.5 * e_tok


def test_error_shrinks_with_window_and_bits():
    w = synth.WORKLOADS["tiny"]
    k, v = synth.kv_tokens(w, 1001, 2001, 1, 256)
    q = synth.queries(w, 1, 256)                    # many queries on the one KV head
    errs = {}
    for fmt in ("int2", "int4", "int8"):
        for r in (0, 128):
            st = cache.build_cache(k, v, _lay(fmt, r=r))
            errs[fmt, r] = _attn_err(st, q, k, v)
    assert errs["int8", 0] < errs["int4", 0] < errs["int2", 0]
    assert errs["int2", 128] < errs["int2", 0] and errs["int4", 128] < errs["int4", 0]


# -------------------------------------------------------------- byte counter
@pytest.mark.parametrize("name,fmt,total", [
    ("llama3_8b", "fp8", 272_891_904), ("llama3_8b", "int8", 338_952_192),
    ("llama3_8b_kivi2", "int2", 140_771_328), ("llama3_70b", "int4", 208_404_480),
    ("long_ctx", "int8", 335_757_312), ("long_ctx", "int4", 201_670_656)])
def test_step_bytes_of_the_workloads(name, fmt, total):
    w = synth.WORKLOADS[name]
    lay = cache.Layout(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, w.seq_len, fmt,
                       residual_tokens=w.residual_tokens, sink_tokens=w.sink_tokens)
    sb = nbytes.step_bytes(lay, w.seq_len)
    assert sb["total"] == total
    # bits per value in the quantized region: codes + fp32 s/z
    bits = 8 * (sb["codes"] + sb["meta"]) / (2 * w.batch * w.num_kv_heads * sb["n_q"] * w.head_dim)
    assert bits == {"fp8": 8, "int8": 10, "int4": 6, "int2": 4}[fmt]


@pytest.mark.parametrize("fmt,bits", [("int8", 9), ("int4", 5), ("int2", 3), ("fp8_e5m2", 8)])
def test_fp16_metadata_and_e5m2_bits_per_value(fmt, bits):
    # one fp16 scale and one fp16 offset per 32 values add 1 bit per value;
    # the 27B study's block formats (one 16-bit scale per 32 values) add 0.5
    w = synth.WORKLOADS["llama3_8b"]
    lay = cache.Layout(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, w.seq_len, fmt,
                       residual_tokens=w.residual_tokens, meta_fp16=fmt != "fp8_e5m2")
    sb = nbytes.step_bytes(lay, w.seq_len)
    got = 8 * (sb["codes"] + sb["meta"]) / (2 * w.batch * w.num_kv_heads * sb["n_q"] * w.head_dim)
    assert got == bits
    assert nbytes.block_bits_per_value(8, 32, 16) + 0.5 == 9


def test_library_side_byte_count_agrees_with_oracle():
    from quantized_kv_cache_quant_amd import accounting
    for name in synth.WORKLOADS:
        w = synth.WORKLOADS[name]
        for fmt, m16, out in (("int8", 0, 0), ("int4", 0, 0), ("int2", 0, 0), ("fp8", 0, 0), ("fp8_e5m2", 0, 0),
                              ("int4", 1, 0), ("int2", 1, 0), ("int4", 0, 1), ("int2", 0, 1), ("int8", 1, 1)):
            for n in (1, 100, w.seq_len, w.seq_len + 37):
                lay = cache.Layout(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, n, fmt,
                                   residual_tokens=w.residual_tokens, sink_tokens=w.sink_tokens,
                                   meta_fp16=bool(m16), outliers=bool(out))
                assert accounting.attention_bytes(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, n, fmt,
                                                  w.sink_tokens, w.residual_tokens, meta_fp16=bool(m16),
                                                  outliers=bool(out)) == nbytes.step_bytes(lay, n)["total"]
