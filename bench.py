"""Decode-step benchmark of the quantized KV cache on one MI355X.

One step = for every layer of the model: append one new token's K / V to
that layer's packed cache (quantize-on-append) and run fused-dequant decode
attention for all query heads, through kv_append_decode_attention (one
split-K attention kernel that also writes the new token into the fp16 ring;
on every 32nd step, when a block leaves the window, the append's kernels
run first).  Inputs
are synthetic and already resident in HBM when the timed region starts.
Each layer owns its own cache buffer, so the timed loop streams every
layer's packed cache from HBM (one layer's cache is larger than the 256 MB
last-level cache, and the 32 layers together are ~8 GB).

Default run (no --workload): the Llama-3-8B layer shape (32 query / 8 KV
heads, head_dim 128) at batch 16 and 8192 cached tokens, 32 layers, with the
cache quantized to INT8 (headline "value") and to FP8 E4M3 ("fp8"); then,
under "workloads", each of the other decode workloads at its own shape and
depth: KIVI-style INT2 on the 8B shape (fp32 scale / zero-point, 128-token
window, one fused one-token append per layer and step, 32 layers), the
Llama-3-70B layer shape in INT4 with 4 fp16 sink tokens (80 layers), and
131072 tokens at batch 1 with INT8 on layers 0-3 and 28-31 and INT4 between
(32 layers); under "tiny_latency" the call latency of the batch-1, 4-query-
head, 256-token INT4 case.  Under "variants" it adds attention-only sweeps of
the 8B shape for the other cache variants (FP8 E5M2; INT8 / INT4 / INT2 with
fp16 scale and offset metadata; INT8 in a paged pool of 32-token pages in
shuffled order; INT8 and INT4 with Keys stored before RoPE, rotated in
attention with base 500000; INT4 and INT2 with one exact fp16 outlier per
group), eight layer caches each.  "cpu_baseline" is the CPU oracle timed on
one layer's decode step of the headline workload on all host cores, and
"pages_context" holds the speed-ups and capacities the pages report, with the
hardware they name, as context (none is this metric on this hardware).

Timed regions, each bracketed by HIP events on the stream the library
launches on (torch's current stream):
  * steps: `--steps` decode steps back to back -> value (effective KV GB/s =
    algorithmic attention bytes / wall time, appends included), ms_per_step,
    tokens/s;
  * prefill: each layer cache's kv_quant_append of the prompt between its own
    event pair -> prefill_quantize (fp16 K/V input GB/s; the first layer's
    call, which pays one-off costs, is left out); flush_traffic_floor_us is
    the library's read-then-write probe (kvq_rw_probe) moving the same
    blocks' bytes with no compute, and frac_of_floor is that time over the
    call's;
  * attention sweep: the kv_decode_attention calls of every layer of one
    format, several rounds back to back between one event pair -> the
    roofline entry (algorithmic bytes per call / mean call time, launch gaps
    included, so the mean is at least the kernel's own duration).  No event
    sits between two calls: each record adds idle time on the stream.
read_gbps_measured is the best rate of the library's plain streaming-read
kernel (kvq_read_probe) over 4 GiB; attn_frac_of_measured_read is the
attention call's rate (roofline.achieved) over it.
roofline.traffic comes from the FETCH_SIZE / WRITE_SIZE counter passes
recorded in profiles/attn_counters.json, scaled by the plain-copy
calibration stored there, and is null when the attention source has changed
since those counters were taken.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "decode-attention effective KV GB/s (% of HBM peak) + tokens/s, batch16 seq8192"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default=None,
                    choices=["llama3_8b", "llama3_8b_kivi2", "llama3_70b", "long_ctx"],
                    help="time one workload only (default: the 8B headline, then every other workload)")
    ap.add_argument("--formats", default=None, help="comma list overriding the workload's formats")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count")
    ap.add_argument("--blocks-per-group", type=int, default=0)
    ap.add_argument("--deterministic", action="store_true",
                    help="time the deterministic hand-out (kv_decode_attention_split, deterministic = 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the attention sweep of the other variants")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--read-sweep", action="store_true",
                    help="only time the plain streaming-read kernel over a range of sizes and print that")
    ap.add_argument("--ingest-counters", metavar="DIR", default=None,
                    help="no GPU work: write profiles/attn_counters.json from the rocprofv3 --pmc runs "
                         "DIR/<key>_FETCH_SIZE and DIR/<key>_WRITE_SIZE (see COUNTER_RUNS)")
    return ap.parse_args()


def read_peak(torch, kvq) -> dict:
    """GB/s of the library's plain streaming-read kernel (kvq_read_probe) over 4 GiB, with one
    and with four workgroups of 512 threads per compute unit (the first is the attention
    kernel's launch shape), each timed with events on the stream it launches on."""
    n = 4 << 30
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4 * cus * 512, dtype=torch.int32, device="cuda")
    res = {}
    for per_cu in (1, 4):
        g = per_cu * cus
        kvq.read_probe(x, sink, g)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            kvq.read_probe(x, sink, g)
        e1.record()
        torch.cuda.synchronize()
        res[f"{per_cu}_per_cu"] = round(n / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9, 1)
    del x, sink
    return res


def copy_bandwidth(torch) -> float:
    """GB/s of a plain device-to-device copy of 2 GiB (read + write bytes)."""
    n = 2 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del x, y
    return 2 * n / (ms * 1e-3) / 1e9


FP8_MAX = {"fp8": 448.0, "fp8_e5m2": 57344.0}
VARIANTS = ("fp8_e5m2", "int8_m16", "int4_m16", "int2_m16", "int8_paged", "int8_rope", "int4_rope", "int4_out",
            "int2_out")
ROPE_THETA = 500000.0


def flush_floor_us(torch, kvq, accounting, w, spec, reps=5) -> float:
    """µs of the library's read-then-write probe (kvq_rw_probe) moving the bytes of the prompt's
    flush in format spec: 32-token blocks of fp16 K and V read whole, then each block's codes and
    metadata written; the same block count as the prompt's kv_quant_append quantizes.  Timed like
    the prefill: one source read by every call, a newly allocated destination per call, one
    event pair per call."""
    fmt, m16, _, _, out = split_spec(spec)
    d = w.head_dim
    read_b = 2 * 32 * d * 2
    pair = 0 if fmt.startswith("fp8") else (4 if m16 else 8) + (4 if out else 0)
    write_b = 2 * 32 * d * accounting.BITS[fmt] // 8 + d * pair + (d // 32) * 32 * pair
    _, nq, _ = accounting.routed(w.seq_len, w.sink_tokens, w.residual_tokens)
    blocks = w.batch * w.num_kv_heads * (nq // 32)
    src = torch.empty(blocks * read_b, dtype=torch.uint8, device="cuda")
    dsts = [torch.empty(blocks * write_b, dtype=torch.uint8, device="cuda") for _ in range(reps + 1)]
    ev = []
    for dst in dsts:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.rw_probe(src, dst, read_b, write_b)
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    us = [1e3 * a.elapsed_time(b) for a, b in ev[1:]]       # the first pays one-off costs
    del src, dsts
    torch.cuda.empty_cache()
    return float(np.mean(us))


def split_spec(spec: str):
    """Format spec -> (kvq format, fp16 metadata, paged, pre-RoPE Keys, outliers): suffix "_m16"
    selects fp16 (s, m) pairs, "_paged" a pool of 32-token pages, "_rope" Keys stored before RoPE,
    "_out" one exact outlier per group."""
    out = spec.endswith("_out")
    spec = spec[:-4] if out else spec
    rope = spec.endswith("_rope")
    spec = spec[:-5] if rope else spec
    paged = spec.endswith("_paged")
    spec = spec[:-6] if paged else spec
    m16 = spec.endswith("_m16")
    return (spec[:-4] if m16 else spec), m16, paged, rope, out


def make_cache(kvq, w, spec, max_tokens, amax_k, amax_v, seed=0):
    import torch
    fmt, m16, paged, rope, out = split_spec(spec)
    # FP8 calibration: amax / (largest finite value) of the prefill, per tensor (a caller input)
    top = FP8_MAX.get(fmt, 448.0)
    pps = max(1, (max_tokens - w.sink_tokens - w.residual_tokens) // 32)   # one block per page
    lay = kvq.make_layout(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, max_tokens, fmt,
                          residual_tokens=w.residual_tokens, sink_tokens=w.sink_tokens,
                          k_scale=np.float32(amax_k / top), v_scale=np.float32(amax_v / top), meta_fp16=m16,
                          page_blocks=1 if paged else 0, num_pages=w.batch * pps if paged else 0,
                          rope_theta=ROPE_THETA if rope else 0.0, outliers=out)
    c = kvq.Cache.create(lay)
    if paged:                                    # every sequence's pages scattered over the pool
        perm = np.random.default_rng(seed).permutation(w.batch * pps).astype(np.int32)
        c.set_block_table(torch.from_numpy(perm.reshape(w.batch, pps)).cuda())
    return c


def call_bytes(accounting, w, spec, n):
    fmt, m16, _, _, out = split_spec(spec)
    return accounting.attention_bytes(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, n, fmt,
                                      w.sink_tokens, w.residual_tokens, meta_fp16=m16, outliers=out)


def back_to_back_us(torch, caches, call, rounds) -> float:
    """Mean µs per call of `rounds` passes of call(c) over the caches, launched back to back
    between one event pair on the launch stream (the launch gaps count; no event record sits
    between two calls, since each record adds idle time on the stream)."""
    for c in caches:                            # one untimed pass
        call(c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        for c in caches:
            call(c)
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / (rounds * len(caches))


def variant_sweep(torch, kvq, synth, accounting, w, specs, args, layers=8, rounds=8):
    """Attention-only timing of each variant: `layers` caches, calls back to back."""
    log(f"variant sweep: generating synthetic prefill for {', '.join(specs)}")
    kp, vp = synth.prefill(w)
    kd = torch.from_numpy(kp).cuda()
    vd = torch.from_numpy(vp).cuda()
    del kp, vp
    amax_k, amax_v = float(kd.abs().max().float().item()), float(vd.abs().max().float().item())
    q = torch.from_numpy(synth.queries(w)).cuda()
    out = torch.empty_like(q)
    res = {}
    for spec in specs:
        caches = []
        for li in range(layers):
            c = make_cache(kvq, w, spec, w.seq_len, amax_k, amax_v, seed=li)
            c.append(kd, vd)
            caches.append(c)
        ws = torch.empty(caches[0].workspace_bytes(args.blocks_per_group) // 4 + 4, dtype=torch.float32,
                         device="cuda")
        us = back_to_back_us(torch, caches, lambda c: c.attention(q, out, ws, args.blocks_per_group), rounds)
        nb = call_bytes(accounting, w, spec, w.seq_len)
        res[spec] = {"attn_call_us": round(us, 2), "bytes_per_attn_call": nb,
                     "attn_gbps": round(nb / (us * 1e-6) / 1e9, 1),
                     "frac_of_hbm_peak": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "layers": layers, "attn_calls_timed": layers * rounds}
        log(f"variant {spec}: attention call {us:.1f} us = {res[spec]['attn_gbps']:.0f} GB/s")
        del caches, ws
        torch.cuda.empty_cache()
    del kd, vd
    torch.cuda.empty_cache()
    return res


def run_format(torch, kvq, synth, accounting, w, fmt_list, args):
    """Time the decode step with the given per-layer formats; returns a result dict."""
    layers = len(fmt_list)
    b, hkv, hq, d, n0 = w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, w.seq_len
    total_steps = args.warmup + args.steps
    max_tokens = n0 + total_steps + 32
    log(f"generating synthetic prefill ({b}x{n0}x{hkv}x{d} fp16 K/V)")
    kp, vp = synth.prefill(w)
    kd = torch.from_numpy(kp).cuda()
    vd = torch.from_numpy(vp).cuda()
    del kp, vp
    amax_k, amax_v = float(kd.abs().max().float().item()), float(vd.abs().max().float().item())
    # every layer's cache is allocated before the first append is timed (an allocation while a
    # kernel runs remaps device memory under it)
    caches = [make_cache(kvq, w, fmt, max_tokens, amax_k, amax_v) for fmt in fmt_list]
    torch.cuda.synchronize()
    pre_ev = []                                 # prefill quantize-on-append, one event pair per layer
    for c in caches:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        c.append(kd, vd)
        e1.record()
        pre_ev.append((e0, e1))
    torch.cuda.synchronize()
    pre_us = [a.elapsed_time(bb) * 1e3 for a, bb in (pre_ev[1:] or pre_ev)]   # the first pays one-off costs
    pre_in = 2 * kd.numel() * kd.element_size()                               # fp16 K and V of the prompt
    floors = {f: flush_floor_us(torch, kvq, accounting, w, f) for f in sorted(set(fmt_list))}
    floor_us = float(np.mean([floors[f] for f in (fmt_list[1:] or fmt_list)]))
    del kd, vd
    log(f"{layers} layer caches prefilled ({sum(c.buf.numel() for c in caches) / 2**30:.2f} GiB)")
    steps_k, steps_v = [], []
    for j in range(total_steps):
        ks, vs = synth.append_step(w, j)
        steps_k.append(torch.from_numpy(ks).cuda())
        steps_v.append(torch.from_numpy(vs).cuda())
    q = torch.from_numpy(synth.queries(w)).cuda()
    out = torch.empty_like(q)
    ws = torch.empty(max(c.workspace_bytes(args.blocks_per_group) for c in caches) // 4 + 4,
                     dtype=torch.float32, device="cuda")

    def step(j):
        # kv_append_decode_attention: append + attention, one launch unless a block leaves the
        # window (every 32nd step); an explicit split takes the two separate calls
        for c in caches:
            if args.blocks_per_group or args.deterministic:
                c.append(steps_k[j], steps_v[j])
                c.attention(q, out, ws, args.blocks_per_group, args.deterministic)
            else:
                c.append_attention(steps_k[j], steps_v[j], q, out, ws)

    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(args.steps):
        step(args.warmup + s)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)

    # attention sweep: the layers of each format, kv_decode_attention calls back to back
    rounds = max(2, args.steps // 8)
    n_final = n0 + total_steps
    by_fmt = {}                                 # per layer format: mean call, bytes, fraction of peak
    for fmt in sorted(set(fmt_list)):
        cf = [c for li, c in enumerate(caches) if fmt_list[li] == fmt]
        us_f = back_to_back_us(torch, cf, lambda c: c.attention(q, out, ws, args.blocks_per_group,
                                                                args.deterministic), rounds)
        nb_f = call_bytes(accounting, w, fmt, n_final)
        by_fmt[fmt] = {"layers": fmt_list.count(fmt), "attn_call_us": round(us_f, 2), "bytes_per_attn_call": nb_f,
                       "attn_gbps": round(nb_f / (us_f * 1e-6) / 1e9, 1),
                       "frac_of_hbm_peak": round(nb_f / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    sweep_bytes = sum(call_bytes(accounting, w, fmt, n_final) for fmt in fmt_list) / layers
    nbytes = 0
    for s in range(args.steps):
        n = n0 + args.warmup + s + 1
        for fmt in fmt_list:
            nbytes += call_bytes(accounting, w, fmt, n)
    ms_step = total_ms / args.steps
    attn_avg_ms = sum(by_fmt[f]["attn_call_us"] for f in fmt_list) / layers / 1e3   # mean over the layers
    res = {
        "formats": sorted(set(fmt_list)),
        "layers": layers,
        "ms_per_step": ms_step,
        "effective_gbps": nbytes / (total_ms * 1e-3) / 1e9,
        "tokens_per_s": b / (ms_step * 1e-3),
        "attn_call_us": attn_avg_ms * 1e3,
        "attn_gbps": sweep_bytes / (attn_avg_ms * 1e-3) / 1e9,
        "step_us_per_layer": ms_step * 1e3 / layers,
        "bytes_per_attn_call": sweep_bytes,
        "attn_calls_timed": rounds * layers,
        "attn_by_format": by_fmt,
        "prefill_quantize": {"us_per_layer": round(float(np.mean(pre_us)), 1),
                             "input_gbps": round(pre_in / (float(np.mean(pre_us)) * 1e-6) / 1e9, 1),
                             "tokens_per_s": round(b * n0 / (float(np.mean(pre_us)) * 1e-6)),
                             "layers_timed": len(pre_us),
                             "flush_traffic_floor_us": round(floor_us, 1),
                             "frac_of_floor": round(floor_us / float(np.mean(pre_us)), 3)},
    }
    res["pct_of_hbm_peak"] = 100.0 * res["effective_gbps"] / HBM_PEAK_GBPS
    log(f"{'/'.join(res['formats'])}: {ms_step:.3f} ms/step, {res['tokens_per_s']:.0f} tok/s, "
        f"effective {res['effective_gbps']:.0f} GB/s; attention call {res['attn_call_us']:.1f} us "
        f"= {res['attn_gbps']:.0f} GB/s")
    del caches, steps_k, steps_v, ws
    torch.cuda.empty_cache()
    return res


COUNTERS_JSON = os.path.join(ROOT, "profiles", "attn_counters.json")
ATTN_SRC = os.path.join(ROOT, "quantized_kv_cache_quant_amd", "csrc", "kvq_attn.hip")
# rocprofv3 --pmc runs read by --ingest-counters: run key -> (bench.py arguments, {entry: kernel
# name filter}); an entry averages the run's attention dispatches whose name holds the filter
COUNTER_RUNS = {
    "llama3_8b": ("--workload llama3_8b --no-variants --no-cpu-baseline --steps 8 --warmup 2",
                  {"int8": "attn_kernel<0", "fp8": "attn_kernel<3"}),
    "kivi2_int2": ("--workload llama3_8b_kivi2 --no-variants --no-cpu-baseline --steps 8 --warmup 2",
                   {"kivi2_int2": "attn_kernel<"}),
    "llama3_70b_int4": ("--workload llama3_70b --no-variants --no-cpu-baseline --steps 8 --warmup 2",
                        {"llama3_70b_int4": "attn_kernel<"}),
    "long_ctx_mixed": ("--workload long_ctx --no-variants --no-cpu-baseline --steps 8 --warmup 2",
                       {"long_ctx_mixed": "attn_kernel<"}),
}


def attn_digest() -> str:
    import hashlib
    return hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()


def counter_traffic(key):
    """Per-call HBM bytes of the attention kernel from profiles/attn_counters.json (entry key:
    a format of the 8B headline or a workload key), or None when the file is absent, has no
    such entry, or was taken on another attention source."""
    try:
        rec = json.load(open(COUNTERS_JSON))
        digest = attn_digest()
    except (OSError, ValueError):
        return None
    if rec.get("kvq_attn_hip_sha256") != digest or key not in rec.get("per_call", {}):
        return None
    c = rec["per_call"][key]
    cal = rec["calibration"]
    return round((c["fetch_kib"] * cal["fetch_factor"] + c["write_kib"] * cal["write_factor"]) * 1024.0)


def read_counter_csv(path):
    """{dispatch id: (kernel name, {counter: value})} of a rocprofv3 counter_collection.csv."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            d = out.setdefault(int(row["Dispatch_Id"]), (row["Kernel_Name"], {}))
            d[1][row["Counter_Name"]] = d[1].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return out


def ingest_counters(root) -> dict:
    """Averages the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) of every run in
    COUNTER_RUNS over its attention dispatches, calibrates both against the run's largest
    plain copy (the 2 GiB device-to-device copy of copy_bandwidth: bytes read, bytes written),
    and writes the record, tied to the attention source's sha256, to profiles/attn_counters.json."""
    import glob
    copy_bytes = float(2 << 30)
    per_call, cal = {}, {"fetch": [], "write": []}
    for key, (_, entries) in COUNTER_RUNS.items():
        vals = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            files = glob.glob(os.path.join(root, f"{key}_{counter}", "**", "*counter_collection.csv"),
                              recursive=True)
            if len(files) != 1:
                raise SystemExit(f"--ingest-counters: expected one counter file for {key} {counter}, "
                                 f"found {files}")
            rows = read_counter_csv(files[0])
            copies = [c.get(counter, 0.0) for name, c in rows.values() if "copyBuffer" in name]
            if not copies:
                raise SystemExit(f"--ingest-counters: no copyBuffer dispatch in {files[0]}")
            cal["fetch" if counter == "FETCH_SIZE" else "write"].append(copy_bytes / (max(copies) * 1024.0))
            for entry, pat in entries.items():
                xs = [c[counter] for name, c in rows.values() if pat in name and counter in c]
                if not xs:
                    raise SystemExit(f"--ingest-counters: no '{pat}' dispatch in {files[0]}")
                vals.setdefault(entry, {})[counter] = (sum(xs) / len(xs), len(xs))
        for entry, v in vals.items():
            per_call[entry] = {"fetch_kib": round(v["FETCH_SIZE"][0], 1), "write_kib": round(v["WRITE_SIZE"][0], 1),
                               "dispatches": v["FETCH_SIZE"][1]}
    # the copy reads and writes 2 GiB: FETCH_SIZE reads half of that on this part (factor 2)
    factors = {k: round(sum(v) / len(v), 3) for k, v in cal.items()}
    rec = {"kvq_attn_hip_sha256": attn_digest(),
           "commands": {k: f"rocprofv3 --pmc <FETCH_SIZE | WRITE_SIZE> --output-format csv -d "
                           f"{root}/{k}_<counter> -o run -- python3 -u bench.py {a}"
                        for k, (a, _) in COUNTER_RUNS.items()},
           "calibration": {"fetch_factor": factors["fetch"], "write_factor": factors["write"],
                           "source": "the largest __amd_rocclr_copyBuffer dispatch of each run: 2 GiB read, "
                                     "2 GiB written"},
           "per_call": per_call}
    with open(COUNTERS_JSON, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def cpu_baseline(w, fmt, seconds):
    """The CPU oracle on one layer's decode step of workload w in format fmt, on all host cores.

    Set-up: the oracle quantizes the prompt plus one appended token of every sequence
    (one thread per sequence; timed as the CPU's prefill quantization).  Timed: the layer's
    decode step as the oracle states it, fp64 dequantization of every (sequence, KV head)
    and fp64 GQA attention of all query heads, one sequence per worker thread, repeated for
    about `seconds`.  The oracle's own functions are called unchanged; the threads only split
    the batch (numpy releases the interpreter lock inside its array operations).  Full-depth
    figures are that one layer's time times the layer count, labelled as extrapolated.
    """
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_info

    from oracle import attention as oattn
    from oracle import cache as ocache
    from oracle import quant
    from quantized_kv_cache_quant_amd import accounting, synth

    cores = len(os.sched_getaffinity(0))
    b = w.batch
    n = w.seq_len + 1
    k, v = synth.prefill(w)
    k1, v1 = synth.append_step(w, 0)
    k = np.concatenate([k, k1], axis=1)
    v = np.concatenate([v, v1], axis=1)
    q = synth.queries(w)
    ks = float(quant.fp8_scale(k)) if fmt.startswith("fp8") else 1.0
    vs = float(quant.fp8_scale(v)) if fmt.startswith("fp8") else 1.0
    lay = ocache.Layout(1, w.num_kv_heads, w.num_q_heads, w.head_dim, n, fmt, residual_tokens=w.residual_tokens,
                        sink_tokens=w.sink_tokens, k_scale=ks, v_scale=vs)
    with ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        states = list(ex.map(lambda i: ocache.build_cache(k[i:i + 1], v[i:i + 1], lay), range(b)))
        t_quant = time.perf_counter() - t0
        del k, v

        def step(i):
            kh, vh = ocache.dequantize(states[i])
            return oattn.attention(q[i:i + 1], kh, vh)

        reps = 0
        t0 = time.perf_counter()
        while True:
            list(ex.map(step, range(b)))
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    layer_s = dt / reps
    nbytes = accounting.attention_bytes(b, w.num_kv_heads, w.num_q_heads, w.head_dim, n, fmt, w.sink_tokens,
                                        w.residual_tokens)
    blas = sorted({(t.get("internal_api"), t.get("num_threads")) for t in threadpool_info()})
    return {"value": round(nbytes / layer_s / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} x one layer's decode step of {w.name} in {fmt} (batch {b}, {n} tokens, "
                      f"{w.num_q_heads}/{w.num_kv_heads} heads): fp64 dequantize + fp64 attention of every "
                      f"(sequence, KV head), one sequence per thread on {cores} threads, {dt:.1f} s",
            "layer_step_s": round(layer_s, 4),
            "tokens_per_s_extrapolated": round(b / (layer_s * w.layers), 3),
            "extrapolation": f"{w.layers} layers x the one-layer step time (not run at full depth)",
            "prefill_quantize_s_per_layer": round(t_quant, 3),
            "prefill_quantize_input_gbps": round(2 * b * w.seq_len * w.num_kv_heads * w.head_dim * 2 / t_quant / 1e9,
                                                 3),
            "os_cpu_count": os.cpu_count(), "affinity_cpus": cores,
            "blas_threads": [{"api": a, "num_threads": t} for a, t in blas]}


def tiny_latency(torch, kvq, synth, calls=200) -> dict:
    """Call latency of the tiny workload (batch 1, 4 query heads on 1 KV head, 256 tokens, INT4,
    32-token window): kv_decode_attention and kv_append_decode_attention, each call between its
    own event pair, and back-to-back calls between one pair (launch-rate bound)."""
    w = synth.WORKLOADS["tiny"]
    k, v = synth.prefill(w)
    lay = kvq.make_layout(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, w.seq_len + calls + 16, "int4",
                          residual_tokens=w.residual_tokens)
    c = kvq.Cache.create(lay)
    c.append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    q = torch.from_numpy(synth.queries(w)).cuda()
    out = torch.empty_like(q)
    ws = torch.empty(c.workspace_bytes(0) // 4 + 4, dtype=torch.float32, device="cuda")
    steps = [synth.append_step(w, j) for j in range(calls)]
    ks = [torch.from_numpy(a).cuda() for a, _ in steps]
    vs = [torch.from_numpy(b).cuda() for _, b in steps]
    for _ in range(10):
        c.attention(q, out, ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for e0, e1 in ev:
        e0.record()
        c.attention(q, out, ws)
        e1.record()
    torch.cuda.synchronize()
    single = 1e3 * float(np.median([a.elapsed_time(b) for a, b in ev]))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        c.attention(q, out, ws)
    e1.record()
    torch.cuda.synchronize()
    b2b = 1e3 * e0.elapsed_time(e1) / calls
    for j, (e0, e1) in enumerate(ev):
        e0.record()
        c.append_attention(ks[j], vs[j], q, out, ws)
        e1.record()
    torch.cuda.synchronize()
    step = 1e3 * float(np.median([a.elapsed_time(b) for a, b in ev]))
    return {"workload": f"tiny: {w.notes}", "attn_call_us": round(single, 2),
            "attn_call_us_back_to_back": round(b2b, 2), "decode_step_us": round(step, 2),
            "calls": calls, "note": "median of per-call event pairs; latency-bound, not a roofline figure"}


def read_sweep(torch, kvq) -> dict:
    """The plain streaming-read kernel (kvq_read_probe, one workgroup of 512 threads per compute
    unit, the attention kernel's launch shape) over a range of sizes: each call reads a fresh
    slice of an 11 GiB buffer (the 256 MB last-level cache cannot serve it), once with each call
    between its own event pair and once with the calls back to back between one pair (the way
    the attention sweep is timed)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    total = 11 << 30
    x = torch.empty(total, dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus * 512, dtype=torch.int32, device="cuda")
    res = {}
    # the attention calls' own sizes (8B INT8 342 MB, FP8 275 MB, KIVI INT2 142 MB, 70B INT4 209 MB,
    # 131k mixed 235 MB mean) among others
    for mb in (64, 128, 142, 209, 235, 275, 342, 1074, 4295):
        nb = mb * 1000000 // 256 * 256
        slices = max(8, min(32, total // nb))
        offs = [(i * nb) % (total - nb + 1) // 256 * 256 for i in range(slices)]
        kvq.read_probe(x[offs[0]:offs[0] + nb], sink, cus)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in offs]
        for (e0, e1), o in zip(ev, offs):
            e0.record()
            kvq.read_probe(x[o:o + nb], sink, cus)
            e1.record()
        torch.cuda.synchronize()
        us = [1e3 * a.elapsed_time(b) for a, b in ev]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for o in offs:
            kvq.read_probe(x[o:o + nb], sink, cus)
        e1.record()
        torch.cuda.synchronize()
        b2b = 1e3 * e0.elapsed_time(e1) / len(offs)
        res[f"{mb}_MB"] = {"mean_us": round(float(np.mean(us)), 2), "min_us": round(float(np.min(us)), 2),
                             "gbps_mean": round(nb / (float(np.mean(us)) * 1e-6) / 1e9, 1),
                             "back_to_back_us": round(b2b, 2), "gbps_back_to_back": round(nb / (b2b * 1e-6) / 1e9, 1),
                             "calls": len(us)}
        log(f"read {mb} MB: {res[f'{mb}_MB']}")
    del x, sink
    return res


PAGES_CONTEXT = {
    "note": "figures the pages report for other kernels on other hardware; context, not this metric",
    "kivi_throughput_speedup": {"value": "2.35-3.47x", "hardware": "not stated on the page",
                                "what": "KIVI 2-bit KV cache (K per channel, V per token, fp16 residual), "
                                        "throughput vs an fp16 cache",
                                "source": "KV Cache Quantization Analysis, sec. 4 (KIVI)"},
    "kvquant_kernel_speedup": {"value": "~1.7x", "hardware": "custom CUDA kernels; GPU not named for this figure",
                               "what": "KVQuant sub-4-bit KV kernels vs fp16",
                               "source": "KV Cache Quantization Analysis, sec. 4 (KVQuant)"},
    "kvquant_context": {"value": "1M tokens on one GPU (10M on 8 GPUs)", "hardware": "one A100-80GB",
                        "what": "KVQuant 3-bit KV cache, LLaMA-7B",
                        "source": "KV Cache Quantization Analysis, sec. 4 (KVQuant)"},
}

# the decode workloads timed after the headline, each at its own shape and depth
OTHER_WORKLOADS = (("kivi2_int2", "llama3_8b_kivi2", ["int2"]), ("llama3_70b_int4", "llama3_70b", ["int4"]),
                   ("long_ctx_mixed", "long_ctx", ["mixed"]))


def layer_formats(w, var, nl):
    if var == "mixed":
        return list(w.formats)[:nl] if nl <= len(w.formats) else (list(w.formats) * nl)[:nl]
    return [var] * nl


def summary(w, r, traffic=None) -> dict:
    """The per-workload entry of the JSON line (traffic: counter HBM bytes per call, or None)."""
    return {"workload": f"{w.name}: {w.notes}", "batch": w.batch, "seq_len": w.seq_len,
            "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "residual_tokens": w.residual_tokens,
            "sink_tokens": w.sink_tokens, "layers": r["layers"], "formats": r["formats"],
            "attn_call_us": round(r["attn_call_us"], 2), "bytes_per_attn_call": r["bytes_per_attn_call"],
            "attn_gbps": round(r["attn_gbps"], 1), "frac_of_hbm_peak": round(r["attn_gbps"] / HBM_PEAK_GBPS, 4),
            "attn_by_format": r["attn_by_format"], "ms_per_step": round(r["ms_per_step"], 4),
            "step_us_per_layer": round(r["step_us_per_layer"], 2), "tokens_per_s": round(r["tokens_per_s"], 1),
            "effective_gbps": round(r["effective_gbps"], 1), "prefill_quantize": r["prefill_quantize"],
            "traffic": traffic}


def main():
    args = parse()
    if args.ingest_counters:
        rec = ingest_counters(args.ingest_counters)
        print(json.dumps(rec["per_call"]), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py: measures one GPU; the decode-attention path shards by KV head or by token "
              "range with no exchange between GPUs, and runs on more than one GPU are not measured here",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from quantized_kv_cache_quant_amd import accounting, kvq, synth
    kvq.lib()
    if args.read_sweep:
        print(json.dumps({"read_probe_sweep": read_sweep(torch, kvq)}), flush=True)
        return
    name = args.workload or "llama3_8b"
    w = synth.WORKLOADS[name]
    if args.formats:
        variants = [f.strip() for f in args.formats.split(",")]
    elif name == "long_ctx":
        variants = ["mixed"]
    elif name == "llama3_8b":
        variants = ["int8", "fp8"]                   # INT8 is the headline line
    else:
        variants = list(w.formats)
    nl = args.layers or w.layers
    results = {}
    for var in variants:
        results[var] = run_format(torch, kvq, synth, accounting, w, layer_formats(w, var, nl), args)
    default_run = args.workload is None and not args.formats and not args.layers
    others = {}
    if default_run:
        for key, wname, fl in OTHER_WORKLOADS:
            wo = synth.WORKLOADS[wname]
            r = run_format(torch, kvq, synth, accounting, wo, layer_formats(wo, fl[0], wo.layers), args)
            others[key] = summary(wo, r, counter_traffic(key))
    vres = None
    if not args.no_variants and name == "llama3_8b" and not args.formats:
        vres = variant_sweep(torch, kvq, synth, accounting, w, VARIANTS, args)
    tiny = tiny_latency(torch, kvq, synth) if default_run else None
    copy_gbps = copy_bandwidth(torch)
    log(f"device-to-device copy: {copy_gbps:.0f} GB/s")
    reads = read_peak(torch, kvq)
    read_gbps = max(reads.values())
    log(f"streaming read (kvq_read_probe, workgroups per compute unit: GB/s): {reads}")
    head = results[variants[0]]
    line = {
        "metric": METRIC,
        "value": round(head["effective_gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{variants[0]} KV codes, f16 MFMA operands, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.notes}", "batch": w.batch, "seq_len": w.seq_len,
                   "layers": head["layers"], "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "residual_tokens": w.residual_tokens,
                   "sink_tokens": w.sink_tokens, "kv_format": variants[0]},
        "tokens_per_s": round(head["tokens_per_s"], 1),
        "pct_of_hbm_peak": round(head["pct_of_hbm_peak"], 2),
        "attn_call_us": round(head["attn_call_us"], 2),
        "step_us_per_layer": round(head["step_us_per_layer"], 2),
        "copy_gbps_measured": round(copy_gbps, 1),
        "read_gbps_measured": read_gbps,
        "read_gbps_by_shape": reads,
        "attn_frac_of_measured_read": round(head["attn_gbps"] / read_gbps, 4),
        "prefill_quantize": head["prefill_quantize"],
        "roofline": {"bound": "hbm", "achieved": round(head["attn_gbps"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(head["attn_gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": counter_traffic(variants[0]),
                     "kernel": "attn_kernel (one kv_decode_attention call, split-K combine in the same kernel)",
                     "bytes_per_launch": head["bytes_per_attn_call"],
                     "call_us": round(head["attn_call_us"], 2)},
    }
    for var in variants[1:]:
        r = results[var]
        line[var] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
        line[var]["traffic"] = counter_traffic(var)
    if others:
        line["workloads"] = others
    if tiny:
        line["tiny_latency"] = tiny
    if vres:
        line["variants"] = vres
    if not args.no_cpu_baseline:
        fmt0 = variants[0] if variants[0] != "mixed" else "int4"
        log(f"timing the CPU oracle on one layer's decode step for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline(w, fmt0, args.cpu_seconds)
    line["pages_context"] = PAGES_CONTEXT
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
