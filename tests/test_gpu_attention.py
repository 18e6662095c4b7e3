"""GPU parity of fused-dequant decode attention vs the fp64 oracle (max-abs 2e-3).

The oracle runs on the cache the library itself produced (read back and
dequantized in fp64), so these tests check the attention arithmetic alone;
the append tests pin the codes.  2e-3 is the tolerance the build targets:
the fp16 output rounding alone contributes up to 2^-11 |out|.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oattn
from oracle import cache as ocache
from oracle import quant
from quantized_kv_cache_quant_amd import kvq, synth

from kvq_testlib import (FP8, append_chunks, assert_states_equal, attention_gpu, check_every_head, make_cache,
                         olayout_of, read_state, require_gpu, split_fmt, to_dev)

pytestmark = pytest.mark.gpu

TOL = 2e-3
W = synth.WORKLOADS


def _oracle_out(c, kw, q):
    st = read_state(c, olayout_of(kw))
    kh, vh = ocache.dequantize(st)
    return oattn.attention(q, kh, vh)


def _kw(name, b, hkv, nrep, maxt, r, s, k, v):
    fmt, m16 = split_fmt(name)
    kw = dict(batch=b, num_kv_heads=hkv, num_q_heads=hkv * nrep, max_tokens=maxt, fmt=fmt,
              residual_tokens=r, sink_tokens=s)
    if m16:
        kw.update(meta_fp16=True)
    if fmt in FP8:
        kw.update(k_scale=float(quant.fp8_scale(k, fmt)), v_scale=float(quant.fp8_scale(v, fmt)))
    return kw


def _build(fmt, b, hkv, nrep, n, r, s, seed=1, w="llama3_8b", chunks=None):
    k, v = synth.kv_tokens(W[w], seed, seed + 1, b, n, hkv, 128)
    if s:                                                      # attention sinks with large logits
        k[:, :s] = (k[:, :s].astype(np.float32) * 10).astype(np.float16)
    kw = _kw(fmt, b, hkv, nrep, n + 64, r, s, k, v)
    c = make_cache(kw)
    append_chunks(c, k, v, chunks or [n])
    q = synth.queries(W[w], b, hkv * nrep, 128, seed_offset=seed)
    return c, kw, q


def test_tiny_workload():
    require_gpu()
    w = W["tiny"]
    k, v = synth.prefill(w)
    kw = dict(batch=1, num_kv_heads=1, num_q_heads=4, max_tokens=256, fmt="int4", residual_tokens=32)
    c = make_cache(kw)
    append_chunks(c, k, v, [256])
    q = synth.queries(w)
    out = attention_gpu(c, q)
    ref = _oracle_out(c, kw, q)
    # the library's cache is the oracle's cache (codes are bit-exact)
    st = ocache.build_cache(k, v, olayout_of(kw))
    kh, vh = ocache.dequantize(st)
    assert np.max(np.abs(oattn.attention(q, kh, vh) - ref)) == 0.0
    assert np.max(np.abs(out.astype(np.float64) - ref)) <= TOL


@pytest.mark.parametrize("fmt", ["int4", "int8", "int2", "fp8", "fp8_e5m2", "int4_m16", "int8_m16", "int2_m16"])
@pytest.mark.parametrize("nrep", [1, 2, 4, 8])
def test_formats_and_gqa(fmt, nrep):
    require_gpu()
    b, hkv, r, s = 2, 2, 32, 0
    n = 32 * 45 + r + 11                                       # 45 blocks: several splits, ragged waves
    c, kw, q = _build(fmt, b, hkv, nrep, n, r, s, seed=nrep)
    out = attention_gpu(c, q)
    ref = _oracle_out(c, kw, q)
    assert np.max(np.abs(out.astype(np.float64) - ref)) <= TOL


@pytest.mark.parametrize("fmt", ["int4", "fp8", "fp8_e5m2", "int2_m16"])
@pytest.mark.parametrize("s,r", [(4, 32), (4, 0), (0, 0), (3, 200)])
def test_sinks_and_windows(fmt, s, r):
    require_gpu()
    n = 32 * 20 + s + r + 3
    c, kw, q = _build(fmt, 2, 2, 4, n, r, s, seed=3)
    out = attention_gpu(c, q)
    ref = _oracle_out(c, kw, q)
    assert np.max(np.abs(out.astype(np.float64) - ref)) <= TOL


@pytest.mark.parametrize("n,s,r", [(1, 0, 32), (3, 4, 32), (5, 4, 0), (31, 0, 0), (32, 0, 0), (33, 0, 0),
                                   (300, 0, 300)])
def test_edge_lengths(n, s, r):
    """Single token, only sinks, only residual, exactly one block, one block + 1."""
    require_gpu()
    c, kw, q = _build("int4", 1, 2, 4, n, r, s, seed=9)
    out = attention_gpu(c, q)
    ref = _oracle_out(c, kw, q)
    assert np.max(np.abs(out.astype(np.float64) - ref)) <= TOL


def test_empty_cache_is_an_error():
    require_gpu()
    kw = dict(batch=1, num_kv_heads=1, num_q_heads=1, max_tokens=64, fmt="int8")
    c = make_cache(kw)
    with pytest.raises(kvq.KvqError) as e:
        attention_gpu(c, np.zeros((1, 1, 128), np.float16))
    assert e.value.status == -8


@pytest.mark.parametrize("fmt", ["int4", "int8", "int2", "fp8", "fp8_e5m2", "int4_m16"])
def test_split_invariance_and_determinism(fmt):
    require_gpu()
    n = 32 * 70 + 40
    c, kw, q = _build(fmt, 2, 2, 4, n, 32, 0, seed=4)
    ref = _oracle_out(c, kw, q)
    outs = {}
    for bpg in (1, 2, 3, 5, 16, 64, 0):          # 1: one block per workgroup; 64: ranges across heads
        for det in (True, False):
            outs[bpg, det] = attention_gpu(c, q, bpg, det).astype(np.float64)
    base = outs[0, True]
    for key, o in outs.items():
        assert np.max(np.abs(o - ref)) <= TOL, key
        # the split changes the fp32 summation order only: at most one fp16 ulp apart
        assert np.all(np.abs(o - base) <= np.maximum(np.abs(base), 1.0) * 2.0**-10), key
    for bpg in (3, 0):
        again = attention_gpu(c, q, bpg, True)
        assert np.array_equal(again.astype(np.float64), outs[bpg, True]), bpg   # bitwise repeatable


@pytest.mark.parametrize("fmt", ["int8", "int2"])
def test_repeated_calls_default_and_deterministic(fmt):
    """Repeatability of the library's own split at a size where every workgroup's wavefronts
    take many blocks: the deterministic mode (static hand-out) repeats bit for bit; the default
    (dynamic hand-out) changes only the fp32 summation order, so repeats stay within one fp16
    ulp of each other and within the bound of the oracle."""
    require_gpu()
    c, kw, q = _build(fmt, 4, 4, 4, 32 * 260 + 45, 128, 0, seed=21)
    ref = _oracle_out(c, kw, q)
    det = [attention_gpu(c, q, 0, True) for _ in range(4)]
    for o in det[1:]:
        assert np.array_equal(o.view(np.uint16), det[0].view(np.uint16))
    base = det[0].astype(np.float64)
    assert np.max(np.abs(base - ref)) <= TOL
    for _ in range(4):
        o = attention_gpu(c, q, 0, False).astype(np.float64)
        assert np.max(np.abs(o - ref)) <= TOL
        assert np.all(np.abs(o - base) <= np.maximum(np.abs(base), 1.0) * 2.0**-10)


def test_arrival_counters_start_and_end_at_zero():
    """The sync plane (one int32 arrival counter per sequence and KV head, through which the
    last workgroup to finish a head takes over its combine) holds garbage before the first
    append, is zeroed by it, and is zero again after every attention call whatever the split;
    the outputs meet the bar each time.  Covers caches with quantized blocks and with the fp16
    segment alone (one workgroup per head, no counters used)."""
    require_gpu()
    # (64, 0): no residual window, and the first append fills two blocks exactly, so it copies
    # no token and launches the copy kernel only to zero the counters
    for n, r in ((32 * 70 + 40, 32), (40, 32), (64, 0)):
        k, v = synth.kv_tokens(W["llama3_8b"], 21, 22, 2, n, 2, 128)
        kw = _kw("int4", 2, 2, 4, n + 64, r, 0, k, v)
        c = make_cache(kw)
        c.plane("sync").fill_(0xA5)
        append_chunks(c, k, v, [n])
        assert not c.plane("sync").cpu().numpy().any(), n
        q = synth.queries(W["llama3_8b"], 2, 8, 128, seed_offset=21)
        ref = _oracle_out(c, kw, q)
        for bpg in (1, 7, 0):
            for det in (True, False):
                o = attention_gpu(c, q, bpg, det).astype(np.float64)
                assert np.max(np.abs(o - ref)) <= TOL, (n, bpg, det)
                assert not c.plane("sync").cpu().numpy().any(), (n, bpg, det)


def test_graph_capture_replays_match_eager():
    """kv_decode_attention captured in a HIP graph (torch.cuda.CUDAGraph on the capture stream)
    and replayed several times, with eager work and a synchronization between replays: every
    replay gives the eager result (bit for bit in deterministic mode, within one fp16 ulp
    otherwise), the arrival counters are back at zero after each replay, and the result meets
    the bar against the oracle.  The call allocates nothing and enqueues only its kernel."""
    require_gpu()
    c, kw, q = _build("int4", 2, 2, 4, 32 * 40 + 20, 32, 0, seed=31)
    ref = _oracle_out(c, kw, q)
    qd = to_dev(q)
    out = torch.empty_like(qd)
    ws = torch.empty(c.workspace_bytes(0) // 4 + 4, dtype=torch.float32, device="cuda")
    counters = lambda: c.plane("sync").cpu().numpy().view(np.int32)
    for det in (True, False):
        c.attention(qd, out, ws, 0, det)
        torch.cuda.synchronize()
        eager = out.cpu().numpy().astype(np.float64)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):                 # warm-up on a side stream before capture
            c.attention(qd, out, ws, 0, det)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c.attention(qd, out, ws, 0, det)
        for rep in range(4):
            out.fill_(float("nan"))                   # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            if det:
                assert np.array_equal(got, eager), rep
            else:
                assert np.all(np.abs(got - eager) <= np.maximum(np.abs(eager), 1.0) * 2.0**-10), rep
            assert np.max(np.abs(got - ref)) <= TOL, rep
            assert not counters().any(), rep
        del g


@pytest.mark.parametrize("fmt,s,r,theta,extra,nrep", [
    ("int4", 0, 32, 0.0, "", 4), ("int8", 4, 32, 0.0, "", 4), ("fp8", 0, 64, 0.0, "", 4),
    ("int2_m16", 0, 32, 0.0, "", 4), ("int4", 2, 32, 500000.0, "", 4), ("int4", 0, 32, 0.0, "outliers", 4),
    ("int8", 3, 32, 0.0, "paged", 4), ("fp8_e5m2", 0, 32, 0.0, "", 8), ("int8_m16", 2, 13, 0.0, "", 1),
    ("int2", 0, 0, 0.0, "", 2)])
def test_fused_append_attention_matches_separate_calls(fmt, s, r, theta, extra, nrep):
    """kv_append_decode_attention (one launch when the token only enters the fp16 ring) against
    kv_quant_append + kv_decode_attention on a twin cache, over 70 one-token decode steps that
    start with sink appends (when S > 0) and cross a block flush (which takes the two-call
    path): every step's
    output agrees within one fp16 ulp (the two runs may hand blocks to wavefronts in different
    orders), some steps are checked against the oracle, and the two caches end bit-identical
    (the fused path's ring copy is exact).  Also with outliers, and for a paged pool (shuffled
    one-block pages; there the whole buffers, pre-filled alike, are compared byte for byte).
    Grouped-query ratios 1, 2, 4 and 8; windows of 0, 13, 32 and 64 tokens."""
    require_gpu()
    b, hkv, n0, steps = 2, 2, 1, 70
    w = W["llama3_8b"]
    k, v = synth.kv_tokens(w, 41, 42, b, n0 + steps, hkv, 128)
    kw = _kw(fmt, b, hkv, nrep, n0 + steps + 8, r, s, k, v)
    if theta:
        kw.update(rope_theta=theta)
    if extra == "outliers":
        kw.update(outliers=1)
    paged = extra == "paged"
    if paged:
        nb = (n0 + steps + 8 - s - r) // 32
        kw.update(page_blocks=1, num_pages=b * nb + 3)
    ca, cb = make_cache(kw), make_cache(kw)
    if paged:
        table = torch.from_numpy(np.random.default_rng(43).permutation(b * nb + 3)[:b * nb]
                                 .reshape(b, nb).astype(np.int32)).cuda()
        for c in (ca, cb):
            c.buf.fill_(0x5A)
            c.set_block_table(table)
    append_chunks(ca, k[:, :n0], v[:, :n0], [n0])
    append_chunks(cb, k[:, :n0], v[:, :n0], [n0])
    ws_bytes = max(ca.workspace_bytes(0), cb.workspace_bytes(0))
    wa = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
    wb = torch.empty_like(wa)
    for i in range(steps):
        kt, vt = to_dev(k[:, n0 + i:n0 + i + 1]), to_dev(v[:, n0 + i:n0 + i + 1])
        q = synth.queries(w, b, hkv * nrep, 128, seed_offset=100 + i)
        qd = to_dev(q)
        oa, ob = torch.empty_like(qd), torch.empty_like(qd)
        ca.append(kt, vt)
        ca.attention(qd, oa, wa)
        cb.append_attention(kt, vt, qd, ob, wb)
        torch.cuda.synchronize()
        a, bb = oa.cpu().numpy().astype(np.float64), ob.cpu().numpy().astype(np.float64)
        assert cb.n_tokens == ca.n_tokens == n0 + i + 1
        assert np.all(np.abs(bb - a) <= np.maximum(np.abs(a), 1.0) * 2.0**-10), i
        if not paged and (i % 17 == 5 or i == steps - 1):
            st = read_state(cb, olayout_of(kw))
            kh, vh = ocache.dequantize(st)
            ref = oattn.attention(q, ocache.attention_keys(st, kh), vh)   # pre-RoPE Keys rotated
            assert np.max(np.abs(bb - ref)) <= TOL, i
    if paged:
        assert torch.equal(ca.buf, cb.buf)
    else:
        olay = olayout_of(kw)
        assert_states_equal(read_state(cb, olay), read_state(ca, olay))


def test_workspace_reuse_any_contents():
    """One workspace, filled with NaN to start with, serves repeated calls and caches of
    other shapes; the deterministic mode repeats bit for bit."""
    require_gpu()
    ca, kwa, qa = _build("int8", 2, 4, 4, 32 * 80 + 7, 32, 0, seed=11)
    cb, kwb, qb = _build("int4", 1, 2, 8, 32 * 300 + 50, 128, 4, seed=12)
    wsb = max(ca.workspace_bytes(5), cb.workspace_bytes(0), ca.workspace_bytes(0))
    ws = torch.full((wsb // 4 + 4,), float("nan"), dtype=torch.float32, device="cuda")
    outs = []
    for c, q, bpg in ((ca, qa, 0), (cb, qb, 0), (ca, qa, 5), (ca, qa, 0), (cb, qb, 0)):
        qd = to_dev(q)
        out = torch.empty_like(qd)
        c.attention(qd, out, ws, bpg, True)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().astype(np.float64))
    assert np.array_equal(outs[0], outs[3]) and np.array_equal(outs[1], outs[4])
    assert np.max(np.abs(outs[0] - _oracle_out(ca, kwa, qa))) <= TOL
    assert np.max(np.abs(outs[1] - _oracle_out(cb, kwb, qb))) <= TOL
    assert np.max(np.abs(outs[2] - outs[0])) <= TOL


def test_closed_forms_on_gpu():
    require_gpu()
    b, hkv, n = 1, 1, 32 * 10 + 32
    # every V row is the same on-grid vector: the output is that vector for any q
    grid = ((np.arange(128) % 16) - 7) * 2.0**-6
    k, _ = synth.kv_tokens(W["llama3_8b"], 5, 6, b, n, hkv, 128)
    v = np.broadcast_to(grid.astype(np.float16), (b, n, hkv, 128)).copy()
    kw = dict(batch=b, num_kv_heads=hkv, num_q_heads=4, max_tokens=n, fmt="int4", residual_tokens=32)
    c = make_cache(kw)
    append_chunks(c, k, v, [n])
    q = synth.queries(W["llama3_8b"], b, 4, 128)
    out = attention_gpu(c, q).astype(np.float64)
    assert np.max(np.abs(out - grid[None, None, :])) <= 2.0**-11
    # q = 0: the mean of the dequantized values
    out0 = attention_gpu(c, np.zeros((b, 4, 128), np.float16)).astype(np.float64)
    assert np.max(np.abs(out0 - _oracle_out(c, kw, np.zeros((b, 4, 128))))) <= TOL


def _full_size(name, fmt, steps=0):
    """Full-size workload in the launch configuration the benchmark times: prefill, `steps`
    one-token appends, one attention call; every (sequence, KV head) pair of the cache is
    compared bit for bit with the oracle's build of the token history, and every output
    element with the fp64 oracle within 2e-3."""
    w = W[name]
    k, v = synth.prefill(w)
    kw = _kw(fmt, w.batch, w.num_kv_heads, w.num_q_heads // w.num_kv_heads, w.seq_len + 64,
             w.residual_tokens, w.sink_tokens, k, v)
    c = make_cache(kw)
    append_chunks(c, k, v, [w.seq_len])
    ks, vs = [k], [v]
    for j in range(steps):
        ka, va = synth.append_step(w, j)
        append_chunks(c, ka, va, [1])
        ks.append(ka)
        vs.append(va)
    q = synth.queries(w)
    out = attention_gpu(c, q)
    check_every_head(c, kw, out, q, np.concatenate(ks, axis=1), np.concatenate(vs, axis=1))


@pytest.mark.parametrize("name,fmt,steps", [("llama3_8b", "fp8", 0), ("llama3_8b", "int8", 0),
                                            ("llama3_8b_kivi2", "int2", 64), ("llama3_70b", "int4", 0),
                                            ("llama3_8b", "fp8_e5m2", 0), ("llama3_70b", "int4_m16", 0),
                                            ("llama3_8b_kivi2", "int2_m16", 0)])
def test_full_size_workloads(name, fmt, steps):
    require_gpu()
    _full_size(name, fmt, steps=steps)


@pytest.mark.parametrize("name,fmt,steps", [("llama3_8b_kivi2", "int2", 64), ("llama3_8b", "int8", 33)])
def test_full_size_fused_decode_steps(name, fmt, steps):
    """The decode step the benchmark times, at full size: after the 8192-token prefill, every
    step goes through kv_append_decode_attention (one launch, or the append's kernels first on
    the step where a block leaves the window); the final cache is compared with the oracle's
    build of the whole token history, and the last step's output with the fp64 oracle, on
    every (sequence, KV head) pair."""
    require_gpu()
    w = W[name]
    k, v = synth.prefill(w)
    kw = _kw(fmt, w.batch, w.num_kv_heads, w.num_q_heads // w.num_kv_heads, w.seq_len + 64,
             w.residual_tokens, w.sink_tokens, k, v)
    c = make_cache(kw)
    append_chunks(c, k, v, [w.seq_len])
    q = synth.queries(w)
    qd = to_dev(q)
    out = torch.empty_like(qd)
    ws = torch.empty(c.workspace_bytes(0) // 4 + 4, dtype=torch.float32, device="cuda")
    for j in range(steps):
        ks, vs = synth.append_step(w, j)
        c.append_attention(to_dev(ks), to_dev(vs), qd, out, ws)
    torch.cuda.synchronize()
    assert c.n_tokens == w.seq_len + steps
    got = out.cpu().numpy()
    kall = np.concatenate([k] + [synth.append_step(w, j)[0] for j in range(steps)], axis=1)
    vall = np.concatenate([v] + [synth.append_step(w, j)[1] for j in range(steps)], axis=1)
    check_every_head(c, kw, got, q, kall, vall)


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_long_context_layer(fmt):
    """batch 1, 131072 tokens: the two layer formats of the mixed-precision stack."""
    require_gpu()
    _full_size("long_ctx", fmt)


@pytest.mark.parametrize("fmt", ["int2", "int4", "int8"])
def test_huge_value_ranges_stay_finite(fmt):
    """Value scales far above 255 (|V| up to ~6e4): P' = p * s must not overflow f16.

    Outputs are thousands in magnitude and come from cancelling sums of
    terms near 1e4, so the check is relative to the output scale (the fp16
    output rounding alone is 2^-11 of it)."""
    require_gpu()
    b, hkv, nrep, n = 1, 2, 4, 32 * 12 + 40
    k, v = synth.kv_tokens(W["llama3_8b"], 21, 22, b, n, hkv, 128)
    v = np.clip(v.astype(np.float32) * 20000.0, -65504, 65504).astype(np.float16)
    kw = dict(batch=b, num_kv_heads=hkv, num_q_heads=hkv * nrep, max_tokens=n, fmt=fmt, residual_tokens=32)
    c = make_cache(kw)
    append_chunks(c, k, v, [n])
    q = synth.queries(W["llama3_8b"], b, hkv * nrep, 128)
    out = attention_gpu(c, q).astype(np.float64)
    ref = _oracle_out(c, kw, q)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - ref)) <= TOL * np.max(np.abs(ref))
