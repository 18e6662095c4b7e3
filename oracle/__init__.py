"""CPU oracle for the quantized KV cache.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
restatement of what the quantized KV cache computes, used to check the HIP
library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  It shares no code with the HIP path
(``quantized_kv_cache_quant_amd``) and imports nothing from it.

Sources (the pages this restates; cited by title and section):

* "KV Cache Quantization Analysis" (ryotta.opik.net, llm_0015) -- the
  technical core: the affine formula (sec. 2), Key per-channel / Value
  per-token and the full-precision recent window (sec. 3), KIVI / FP8 / mixed
  precision (sec. 4), quantize-on-write / dequantize-before-attention
  (sec. 5) and the KV_bytes formula (the "memory-size sense" box).
* "W4A16 + KV cache quantization: combined accuracy" (hrletsgo.me) -- the
  70B worked example of the KV size (section on the dual memory pressure),
  the scaled softmax (section on where the errors meet) and attention sinks
  (section on layer sensitivity).
* The community KLD study of KV-cache quantization on a 27B model
  (molayo1419.me) -- the per-token cache-size table.

Modules
-------
quant      integer affine group quantization (fp32-exact) and OCP FP8 E4M3.
cache      token routing: sinks, quantized body, fp16 residual window.
layout     the library's documented byte layout, restated for comparison.
attention  fp64 GQA decode attention over the dequantized cache.
rope       rotary position embedding of pre-RoPE Keys (fp64).
nbytes     the KV_bytes formula and per-step algorithmic byte counts.

Parity status: every function is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` except the page's quality numbers (perplexity,
KL divergence, GSM8K), which need models and datasets and stay
"parity unpinned".
"""
