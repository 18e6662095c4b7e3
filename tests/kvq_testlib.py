"""Helpers shared by the GPU parity tests: drive the library, read its planes back.

Reading back uses the oracle's restatement of the documented byte layout
(``oracle.layout``) to turn the library's raw planes into logical codes,
scales and zero-points; the oracle's own quantization of the same inputs is
computed by ``oracle.cache.build_cache``.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from oracle import attention as oattn
from oracle import cache as ocache
from oracle import layout as olayout
from quantized_kv_cache_quant_amd import kvq

BITS = {"int8": 8, "int4": 4, "int2": 2, "fp8": 8, "fp8_e5m2": 8}
FP8 = ("fp8", "fp8_e5m2")


def split_fmt(name: str):
    """Test format names: a kvq format, with suffix "_m16" for fp16 metadata."""
    return (name[:-4], True) if name.endswith("_m16") else (name, False)


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    kvq.lib()                      # raises if libkvq.so is missing


def olayout_of(lay_kw: dict) -> ocache.Layout:
    k = dict(lay_kw)
    return ocache.Layout(k["batch"], k["num_kv_heads"], k["num_q_heads"], 128, k["max_tokens"], k["fmt"],
                         residual_tokens=k.get("residual_tokens", 128), sink_tokens=k.get("sink_tokens", 0),
                         k_scale=k.get("k_scale", 1.0), v_scale=k.get("v_scale", 1.0),
                         meta_fp16=bool(k.get("meta_fp16", False)), rope_theta=float(k.get("rope_theta", 0.0)),
                         outliers=bool(k.get("outliers", False)))


CANARY = 0xC5          # guard byte pattern
GUARD = 256            # guard bytes after the cache buffer, the workspace and the output


def make_cache(lay_kw: dict) -> kvq.Cache:
    """A cache whose device buffer is followed by GUARD canary bytes (and pre-filled with the
    canary, so the alignment gaps between planes hold it too); see check_guards."""
    k = dict(lay_kw)
    lay = kvq.make_layout(k.pop("batch"), k.pop("num_kv_heads"), k.pop("num_q_heads"), 128,
                          k.pop("max_tokens"), k.pop("fmt"), **k)
    nbytes = kvq.cache_bytes(lay)
    full = torch.full((nbytes + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
    buf = full[:nbytes]                      # torch's allocations are 512-byte aligned
    h = kvq.CacheStruct()
    kvq.check(kvq.lib().kvq_cache_init(ctypes.byref(h), ctypes.byref(lay), ctypes.c_void_p(buf.data_ptr()), nbytes),
              "kvq_cache_init")
    c = kvq.Cache(lay, buf, h)
    c.guard = full[nbytes:]
    return c


def plane_gaps(c: kvq.Cache):
    """Byte ranges of the cache buffer that belong to no plane (alignment padding)."""
    spans = sorted((c.handle.plane_off[i], c.handle.plane_off[i] + c.handle.plane_bytes[i])
                   for i in range(len(kvq.PLANES)))
    gaps, end = [], 0
    for a, b in spans:
        if a > end:
            gaps.append((end, a))
        end = max(end, b)
    if end < c.buf.numel():
        gaps.append((end, c.buf.numel()))
    return gaps


def check_guards(c: kvq.Cache) -> None:
    """No write past the cache buffer (the trailing canary bytes) and none into the padding
    between planes (every padding byte still holds the one value it was filled with)."""
    g = getattr(c, "guard", None)
    if g is not None:
        assert bool((g == CANARY).all()), "a kernel wrote past the end of the cache buffer"
    gaps = plane_gaps(c)
    if gaps:
        pad = torch.cat([c.buf[a:b] for a, b in gaps])
        assert bool((pad == pad[0]).all()), "a kernel wrote into the padding between planes"


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def append_chunks(c: kvq.Cache, k: np.ndarray, v: np.ndarray, chunks) -> None:
    """Append k, v [B][n][Hkv][D] in the given chunk sizes."""
    t0 = 0
    for t in chunks:
        c.append(to_dev(k[:, t0:t0 + t]), to_dev(v[:, t0:t0 + t]))
        t0 += t
    assert t0 == k.shape[1]
    torch.cuda.synchronize()
    check_guards(c)


def plane_np(c: kvq.Cache, name: str) -> np.ndarray:
    return c.plane(name).cpu().numpy()


def read_state(c: kvq.Cache, olay: ocache.Layout) -> ocache.CacheState:
    """The library's cache contents as a logical oracle.CacheState."""
    b, hkv, d = olay.batch, olay.num_kv_heads, 128
    bits = BITS[olay.fmt]
    nb_cap = c.handle.n_blocks_cap
    rs = c.handle.ring_slots
    n = c.n_tokens
    n_sink, n_q, r = c.window()
    nb = n_q // 32
    row = d * bits // 8

    def pl(name, dtype, shape):
        return plane_np(c, name).view(dtype).reshape(shape)

    pb = c.handle.layout.page_blocks
    if pb > 0:                                   # paged: gather the logical blocks through the table
        recs = c.handle.layout.num_pages * hkv * pb
        table = c.table.cpu().numpy()

        def blocks(name, dtype, shape):
            return olayout.gather_paged(pl(name, dtype, (recs,) + shape), table, hkv, pb, nb)
    else:
        def blocks(name, dtype, shape):
            return pl(name, dtype, (b, hkv, nb_cap) + shape)[:, :, :nb]
    kc = blocks("k_codes", np.uint8, (32 * row,))
    vc = blocks("v_codes", np.uint8, (32 * row,))
    rope = olay.rope_theta > 0
    codes_k = olayout.unpack_k_codes(kc, olay.fmt, d, rope=rope)
    codes_v = olayout.unpack_v_codes(vc, olay.fmt, d)
    s_k = z_k = s_v = z_v = None
    if olay.fmt not in FP8:
        mt = np.float16 if olay.meta_fp16 else np.float32
        km = blocks("k_meta", mt, (d, 2))
        vm = blocks("v_meta", mt, (4, 32, 2))
        s_k, z_k = olayout.unpack_k_meta(km, rope=rope)
        s_v, z_v = olayout.unpack_v_meta(vm)
        if olay.outliers:
            ko = blocks("k_out", np.uint32, (d,))
            vo = blocks("v_out", np.uint32, (4, 32))
            ko_i, ko_v = olayout.unpack_outliers(ko)
            vo_i, vo_v = olayout.unpack_v_outliers(vo)
    ring_k = pl("k_ring", np.float16, (b, hkv, rs, d))
    ring_v = pl("v_ring", np.float16, (b, hkv, rs, d))
    slots = (np.arange(n_q, n_q + r) % rs).astype(np.int64)
    s_cap = olay.sink_tokens
    if s_cap:
        sk = pl("k_sink", np.float16, (b, hkv, s_cap, d))[:, :, :n_sink]
        sv = pl("v_sink", np.float16, (b, hkv, s_cap, d))[:, :, :n_sink]
    else:
        sk = sv = np.zeros((b, hkv, 0, d), np.float16)
    st = ocache.CacheState(olay, n, n_sink, n_q, r, sk.copy(), sv.copy(), codes_k, codes_v, s_k, z_k, s_v,
                           z_v, ring_k[:, :, slots].copy(), ring_v[:, :, slots].copy(), slots)
    if olay.outliers and olay.fmt not in FP8:
        st.ko_idx, st.ko_val, st.vo_idx, st.vo_val = ko_i, ko_v, vo_i, vo_v
    return st


def assert_states_equal(got: ocache.CacheState, exp: ocache.CacheState, heads=None) -> None:
    """Bitwise equality of codes, scales, zero-points, residual and sinks."""
    assert (got.n_sink, got.n_q, got.r) == (exp.n_sink, exp.n_q, exp.r)
    sel = (slice(None), slice(None)) if heads is None else tuple(np.array(heads).T)

    def eq(a, b, what):
        if a is None and b is None:
            return
        a = np.asarray(a)[sel]
        b = np.asarray(b)[sel]
        if a.dtype.kind == "f":
            a = a.view(np.uint32 if a.dtype == np.float32 else np.uint16)
            b = b.view(np.uint32 if b.dtype == np.float32 else np.uint16)
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"

    eq(got.codes_k, exp.codes_k, "K codes")
    eq(got.codes_v, exp.codes_v, "V codes")
    eq(got.s_k, exp.s_k, "K scale")
    eq(got.z_k, exp.z_k, "K zero-point")
    eq(got.s_v, exp.s_v, "V scale")
    eq(got.z_v, exp.z_v, "V zero-point")
    eq(got.res_k, exp.res_k, "K residual")
    eq(got.res_v, exp.res_v, "V residual")
    eq(got.sink_k, exp.sink_k, "K sinks")
    eq(got.sink_v, exp.sink_v, "V sinks")
    eq(got.ko_idx, exp.ko_idx, "K outlier index")
    eq(got.ko_val, exp.ko_val, "K outlier value")
    eq(got.vo_idx, exp.vo_idx, "V outlier index")
    eq(got.vo_val, exp.vo_val, "V outlier value")


def attention_gpu(c: kvq.Cache, q: np.ndarray, blocks_per_group: int = 0,
                  deterministic: bool = False) -> np.ndarray:
    """One attention call with guard bytes after the output and the workspace; the cache itself
    must come out unchanged apart from its sync plane (attention only reads it)."""
    qd = to_dev(q)
    n_out = qd.numel()
    out_full = torch.full((n_out + GUARD // 2,), float("nan"), dtype=torch.float16, device="cuda")
    out = out_full[:n_out].view(qd.shape)
    need = c.workspace_bytes(blocks_per_group)
    ws_full = torch.full((need + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
    ws = ws_full[:need]
    so, sb = c.handle.plane_off[kvq.PLANES.index("sync")], c.handle.plane_bytes[kvq.PLANES.index("sync")]
    before = c.buf.clone()
    c.attention(qd, out, ws, blocks_per_group, deterministic)
    torch.cuda.synchronize()
    assert torch.isnan(out_full[n_out:]).all(), "attention wrote past its output"
    assert bool((ws_full[need:] == CANARY).all()), "attention wrote past its workspace"
    after = c.buf
    assert torch.equal(before[:so], after[:so]) and torch.equal(before[so + sb:], after[so + sb:]), \
        "attention changed the cache outside its sync plane"
    check_guards(c)
    del before
    return out.cpu().numpy()


def substate(st: ocache.CacheState, bi: int, gi: int | None = None) -> ocache.CacheState:
    """The (sequence bi, KV head gi) slice of a cache state, as a 1 x 1 state; with gi None,
    sequence bi with all its KV heads."""
    hs = slice(None) if gi is None else slice(gi, gi + 1)

    def cut(a):
        return None if a is None else a[bi:bi + 1, hs]
    lay = st.layout
    hkv = lay.num_kv_heads if gi is None else 1
    sub = ocache.Layout(1, hkv, lay.n_rep * hkv, lay.head_dim, lay.max_tokens, lay.fmt, lay.k_group_tokens,
                        lay.v_group_channels, lay.residual_tokens, lay.sink_tokens, lay.k_scale, lay.v_scale,
                        lay.meta_fp16, lay.rope_theta, lay.outliers)
    return ocache.CacheState(sub, st.n, st.n_sink, st.n_q, st.r, cut(st.sink_k), cut(st.sink_v),
                             cut(st.codes_k), cut(st.codes_v), cut(st.s_k), cut(st.z_k), cut(st.s_v),
                             cut(st.z_v), cut(st.res_k), cut(st.res_v), st.res_slots, cut(st.ko_idx),
                             cut(st.ko_val), cut(st.vo_idx), cut(st.vo_val))


def check_every_head(c: kvq.Cache, kw: dict, out: np.ndarray, q: np.ndarray, k: np.ndarray | None = None,
                     v: np.ndarray | None = None, tol: float = 2e-3) -> float:
    """Parity of a whole cache and one attention output, every (sequence, KV head) pair.

    With the token history k, v [B][n][Hkv][D] the library's codes, scales, zero-points,
    residual ring and sinks must equal the oracle's build of that history bit for bit;
    then every element of ``out`` [B][Hq][D] must lie within ``tol`` of the fp64 oracle's
    attention over the library's own cache (dequantized exactly, rotated for pre-RoPE
    Keys).  Works one sequence at a time to bound host memory.  Returns the max-abs error.
    """
    olay = olayout_of(kw)
    st = read_state(c, olay)
    if k is not None:
        assert_states_equal(st, ocache.build_cache(k, v, olay))
    worst = 0.0
    for bi in range(olay.batch):
        one = substate(st, bi)
        kh, vh = ocache.dequantize(one)
        ref = oattn.attention(q[bi:bi + 1], ocache.attention_keys(one, kh), vh)
        err = np.abs(out[bi:bi + 1].astype(np.float64) - ref)
        worst = max(worst, float(err.max()))
        assert err.max() <= tol, (bi, np.unravel_index(int(err.argmax()), err.shape), float(err.max()))
    assert np.all(np.isfinite(out))
    return worst
