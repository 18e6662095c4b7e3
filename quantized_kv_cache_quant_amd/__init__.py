"""Quantized KV cache for MI355X (gfx950): quantize-on-append + fused-dequant decode attention.

Submodules (imported on demand, so that ``synth`` works without the built library):

* ``kvq``    -- ctypes binding of ``libkvq.so`` (C ABI in ``include/kvq.h``)
* ``synth``  -- seeded synthetic workloads (shapes of the Llama-3 layers)
* ``build``  -- hipcc build of ``libkvq.so`` for gfx950
"""
__all__ = ["kvq", "synth", "build"]
