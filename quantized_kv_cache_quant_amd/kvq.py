"""ctypes binding of ``libkvq.so`` (the C ABI declared in ``include/kvq.h``).

Argument marshalling only: every step of quantization and attention runs in
the library's HIP kernels.  torch tensors supply device memory and the
current HIP stream.  Importing this module without a built library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

# KVQ_LIBRARY overrides the path (e.g. the host-sanitizer build that the CPU ABI tests load)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_OK = 0
STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_NULL", -2: "KVQ_ERR_LAYOUT", -3: "KVQ_ERR_UNSUPPORTED",
          -4: "KVQ_ERR_CAPACITY", -5: "KVQ_ERR_ALIGN", -6: "KVQ_ERR_WORKSPACE", -7: "KVQ_ERR_HIP",
          -8: "KVQ_ERR_EMPTY"}
FORMATS = {"int8": 0, "int4": 1, "int2": 2, "fp8": 3, "fp8_e5m2": 4}
PLANES = ("k_codes", "v_codes", "k_meta", "v_meta", "k_ring", "v_ring", "k_sink", "v_sink", "k_out", "v_out",
          "sync")
EXPORTS = ("kvq_status_string", "kvq_layout_validate", "kvq_cache_bytes", "kvq_cache_init",
           "kvq_cache_plane", "kvq_cache_window", "kv_quant_append", "kvq_workspace_bytes",
           "kv_decode_attention", "kv_decode_attention_split", "kvq_cache_set_block_table",
           "kvq_read_probe", "kvq_rw_probe", "kv_append_decode_attention", "kv_decode_attention_noalloc")


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class Layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("format", ctypes.c_int32),
                ("k_group_tokens", ctypes.c_int32), ("v_group_channels", ctypes.c_int32),
                ("residual_tokens", ctypes.c_int32), ("sink_tokens", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float), ("meta_fp16", ctypes.c_int32),
                ("page_blocks", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("outliers", ctypes.c_int32)]


class CacheStruct(ctypes.Structure):
    _fields_ = [("layout", Layout), ("base", ctypes.c_void_p), ("bytes", ctypes.c_uint64),
                ("n_tokens", ctypes.c_int64), ("n_blocks_cap", ctypes.c_int32),
                ("ring_slots", ctypes.c_int32), ("plane_off", ctypes.c_uint64 * len(PLANES)),
                ("plane_bytes", ctypes.c_uint64 * len(PLANES)), ("block_table", ctypes.c_void_p),
                ("table_stride", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run quantized_kv_cache_quant_amd.build first")
        # torch ships its own HIP runtime; load it first so that the library
        # binds to the runtime that owns torch's memory and streams (the
        # other order leaves two runtimes in the process and torch's kernel
        # launches fail with "invalid device function")
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, I32, U64, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_int64
        LP, CP = ctypes.POINTER(Layout), ctypes.POINTER(CacheStruct)
        sig = {
            "kvq_status_string": (ctypes.c_char_p, [I32]),
            "kvq_layout_validate": (I32, [LP]),
            "kvq_cache_bytes": (I32, [LP, ctypes.POINTER(U64)]),
            "kvq_cache_init": (I32, [CP, LP, P, U64]),
            "kvq_cache_plane": (I32, [CP, I32, ctypes.POINTER(U64), ctypes.POINTER(U64)]),
            "kvq_cache_window": (I32, [CP, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64)]),
            "kv_quant_append": (I32, [CP, P, P, I32, P]),
            "kvq_workspace_bytes": (I32, [CP, I32, ctypes.POINTER(U64)]),
            "kv_decode_attention": (I32, [CP, P, P, P, U64, P]),
            "kv_decode_attention_split": (I32, [CP, P, P, P, U64, I32, I32, P]),
            "kvq_cache_set_block_table": (I32, [CP, P, I32]),
            "kvq_read_probe": (I32, [P, U64, P, U64, I32, P]),
            "kvq_rw_probe": (I32, [P, U64, P, U64, ctypes.c_uint32, ctypes.c_uint32, P]),
            "kv_append_decode_attention": (I32, [CP, P, P, P, P, P, U64, P]),
            "kv_decode_attention_noalloc": (I32, [CP, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int, where: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, where)


def make_layout(batch, num_kv_heads, num_q_heads, head_dim, max_tokens, fmt, *, k_group_tokens=32,
                v_group_channels=32, residual_tokens=128, sink_tokens=0, k_scale=1.0, v_scale=1.0,
                meta_fp16=False, page_blocks=0, num_pages=0, rope_theta=0.0, outliers=False) -> Layout:
    return Layout(batch, num_kv_heads, num_q_heads, head_dim, max_tokens, FORMATS[fmt], k_group_tokens,
                  v_group_channels, residual_tokens, sink_tokens, float(k_scale), float(v_scale), int(meta_fp16),
                  int(page_blocks), int(num_pages), float(rope_theta), int(outliers))


def cache_bytes(layout: Layout) -> int:
    n = ctypes.c_uint64()
    check(lib().kvq_cache_bytes(ctypes.byref(layout), ctypes.byref(n)), "kvq_cache_bytes")
    return n.value


def _stream(stream) -> ctypes.c_void_p:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Cache:
    """One layer's packed cache: a device byte tensor plus the host handle."""
    layout: Layout
    buf: "object"          # torch.uint8 device tensor (keeps the memory alive)
    handle: CacheStruct
    table: "object" = None  # paged caches: the bound int32 block table (kept alive here)

    @classmethod
    def create(cls, layout: Layout, device="cuda") -> "Cache":
        import torch
        nbytes = cache_bytes(layout)
        # 256-byte alignment: torch's caching allocator returns 512-byte aligned blocks
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        h = CacheStruct()
        check(lib().kvq_cache_init(ctypes.byref(h), ctypes.byref(layout), ctypes.c_void_p(buf.data_ptr()),
                                   nbytes), "kvq_cache_init")
        return cls(layout, buf, h)

    @property
    def n_tokens(self) -> int:
        return self.handle.n_tokens

    def window(self):
        a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        check(lib().kvq_cache_window(ctypes.byref(self.handle), ctypes.byref(a), ctypes.byref(b),
                                     ctypes.byref(c)), "kvq_cache_window")
        return a.value, b.value, c.value

    def plane(self, name: str):
        """A uint8 view of one plane of the device buffer."""
        off, nb = ctypes.c_uint64(), ctypes.c_uint64()
        check(lib().kvq_cache_plane(ctypes.byref(self.handle), PLANES.index(name), ctypes.byref(off),
                                    ctypes.byref(nb)), "kvq_cache_plane")
        return self.buf[off.value:off.value + nb.value]

    def set_block_table(self, table) -> None:
        """Paged caches: bind an int32 device tensor [B][stride] of page ids (None unbinds)."""
        import torch
        if table is None:
            check(lib().kvq_cache_set_block_table(ctypes.byref(self.handle), None, 0), "kvq_cache_set_block_table")
            self.table = None
            return
        if not table.is_cuda or table.dtype != torch.int32 or table.dim() != 2 or not table.is_contiguous():
            raise ValueError("block table must be a contiguous int32 device tensor [B][stride]")
        check(lib().kvq_cache_set_block_table(ctypes.byref(self.handle), ctypes.c_void_p(table.data_ptr()),
                                              int(table.shape[1])), "kvq_cache_set_block_table")
        self.table = table

    def _check_kv(self, k, v, t=None) -> int:
        """k, v: fp16 device tensors of one shape [B][T][Hkv][D] matching the layout; returns T.
        Shapes are checked first, then dtype, contiguity and device: a mistake raises ValueError
        before anything reaches the library."""
        L = self.layout
        if k.dim() != 4 or tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"K and V must both be [B][T][Hkv][D]; got {tuple(k.shape)} and {tuple(v.shape)}")
        if (k.shape[0], k.shape[2], k.shape[3]) != (L.batch, L.num_kv_heads, L.head_dim):
            raise ValueError(f"K / V shape {tuple(k.shape)} does not match the layout "
                             f"[{L.batch}][T][{L.num_kv_heads}][{L.head_dim}]")
        if t is not None and k.shape[1] != t:
            raise ValueError(f"K / V must hold {t} token(s) per sequence; got {k.shape[1]}")
        _check_tensor(k, "K")
        _check_tensor(v, "V")
        return int(k.shape[1])

    def _check_q_out(self, q, out, ws) -> None:
        """q, out: fp16 device tensors [B][Hq][D]; ws: a device tensor (shapes checked first)."""
        L = self.layout
        want = (L.batch, L.num_q_heads, L.head_dim)
        for t, name in ((q, "q"), (out, "out")):
            if tuple(t.shape) != want:
                raise ValueError(f"{name} must be [{want[0]}][{want[1]}][{want[2]}]; got {tuple(t.shape)}")
        _check_tensor(q, "q")
        _check_tensor(out, "out")
        if not getattr(ws, "is_cuda", False):
            raise ValueError("ws must be a device tensor")

    def append(self, k, v, stream=None) -> None:
        """k, v: contiguous fp16 device tensors [B][T][Hkv][D]."""
        t = self._check_kv(k, v)
        check(lib().kv_quant_append(ctypes.byref(self.handle), ctypes.c_void_p(k.data_ptr()),
                                    ctypes.c_void_p(v.data_ptr()), int(t), _stream(stream)), "kv_quant_append")

    def append_attention(self, k, v, q, out, ws, stream=None) -> None:
        """One decode step (kv_append_decode_attention): k, v fp16 [B][1][Hkv][D]; q, out fp16
        [B][Hq][D]; ws: device scratch tensor."""
        self._check_kv(k, v, 1)
        self._check_q_out(q, out, ws)
        check(lib().kv_append_decode_attention(ctypes.byref(self.handle), ctypes.c_void_p(k.data_ptr()),
                                               ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                               ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                               ws.numel() * ws.element_size(), _stream(stream)),
              "kv_append_decode_attention")

    def workspace_bytes(self, blocks_per_group: int = 0) -> int:
        n = ctypes.c_uint64()
        check(lib().kvq_workspace_bytes(ctypes.byref(self.handle), int(blocks_per_group), ctypes.byref(n)),
              "kvq_workspace_bytes")
        return n.value

    def attention(self, q, out, ws, blocks_per_group: int = 0, deterministic: bool = False,
                  stream=None) -> None:
        """q, out: contiguous fp16 device tensors [B][Hq][D]; ws: device scratch tensor."""
        self._check_q_out(q, out, ws)
        check(lib().kv_decode_attention_split(ctypes.byref(self.handle), ctypes.c_void_p(q.data_ptr()),
                                              ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                              ws.numel() * ws.element_size(), int(blocks_per_group),
                                              int(bool(deterministic)), _stream(stream)),
              "kv_decode_attention")


    def attention_noalloc(self, q, out, stream=None) -> None:
        """kv_decode_attention_noalloc: q, out contiguous fp16 device tensors [B][Hq][D]; the
        partials go to the library's own per-GPU workspace (nothing is allocated)."""
        L = self.layout
        want = (L.batch, L.num_q_heads, L.head_dim)
        for t, name in ((q, "q"), (out, "out")):
            if tuple(t.shape) != want:
                raise ValueError(f"{name} must be [{want[0]}][{want[1]}][{want[2]}]; got {tuple(t.shape)}")
        _check_tensor(q, "q")
        _check_tensor(out, "out")
        check(lib().kv_decode_attention_noalloc(ctypes.byref(self.handle), ctypes.c_void_p(q.data_ptr()),
                                                ctypes.c_void_p(out.data_ptr()), _stream(stream)),
              "kv_decode_attention_noalloc")


def _check_tensor(t, name: str) -> None:
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != torch.float16 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float16 tensor")


def read_probe(buf, sink, groups: int = 0, stream=None) -> None:
    """Diagnostic streaming read of a device tensor (see kvq_read_probe): buf is read whole;
    sink is a device tensor of at least 4 * 512 * groups bytes (groups 0: one workgroup per
    compute unit)."""
    check(lib().kvq_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                               ctypes.c_void_p(sink.data_ptr()), sink.numel() * sink.element_size(),
                               int(groups), _stream(stream)), "kvq_read_probe")


def rw_probe(src, dst, read_bytes: int, write_bytes: int, stream=None) -> None:
    """Diagnostic read-then-write traffic of a flush (see kvq_rw_probe): src (device tensor)
    is read whole in units of read_bytes; dst receives write_bytes per unit."""
    check(lib().kvq_rw_probe(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                             ctypes.c_void_p(dst.data_ptr()), dst.numel() * dst.element_size(),
                             int(read_bytes), int(write_bytes), _stream(stream)), "kvq_rw_probe")
