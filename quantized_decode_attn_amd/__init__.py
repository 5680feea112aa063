"""Python binding of libkvq (2/3/4-bit KV-cache quantization and decode attention over
the packed cache, HIP kernels for gfx950).

Argument marshalling only: every step of the path runs inside libkvq.so.  PyTorch
provides device memory and the current stream.  If the library has not been built
every call raises: there is no fallback.

The functions carry the names of the C ABI in ``include/kvq.h``
(``kvq_cache_layout``, ``kvq_cache_init``, ``kvq_quantize_append``,
``kvq_decode_workspace_bytes``, ``kvq_decode_attention``, ``kvq_decode_attention_noalloc``,
``kvq_chunk_workspace_bytes``, ``kvq_chunk_attention``, ``kvq_decode_step``, ``kvq_dequantize``,
``kvq_status_string``); ``Cache`` bundles the buffers of one cache.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ECAPACITY, KVQ_EWORKSPACE, KVQ_EHIP = 0, -1, -2, -3, -4, -5
EXPORTED = ["kvq_status_string", "kvq_cache_layout", "kvq_cache_init", "kvq_quantize_append",
            "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_decode_attention_noalloc",
            "kvq_chunk_workspace_bytes", "kvq_chunk_attention", "kvq_decode_step", "kvq_dequantize",
            "kvq_paged_layout", "kvq_quantize_append_seqs"]
NOALLOC_SCRATCH_BYTES = 16 << 20   # KVQ_NOALLOC_SCRATCH_BYTES


class KvqConfig(C.Structure):
    _fields_ = [("batch", C.c_int32), ("q_heads", C.c_int32), ("kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("capacity", C.c_int32), ("k_bits", C.c_int32),
                ("k_mode", C.c_int32), ("k_block", C.c_int32), ("v_bits", C.c_int32),
                ("v_group", C.c_int32), ("clip_quantile", C.c_float), ("outlier_pct", C.c_int32),
                ("rope_theta", C.c_float), ("keep_pct", C.c_int32), ("v_mode", C.c_int32)]


BUFFERS = ["k_codes", "k_scale", "k_zero", "k_lut", "k_tail", "v_codes", "v_scale", "v_zero",
           "v_tail", "k_rowptr", "k_col", "k_val", "v_rowptr", "v_col", "v_val", "rope",
           "k_keep_idx", "k_keep_val", "v_lut"]


class KvqLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in BUFFERS]


class KvqCache(C.Structure):
    _fields_ = ([("cfg", KvqConfig), ("length", C.c_int64)] + [(n, C.c_void_p) for n in BUFFERS] +
                [("block_table", C.c_void_p), ("num_blocks", C.c_int32), ("seq_lens", C.c_void_p),
                 ("seq_lens_host", C.POINTER(C.c_int64))])


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s (status %d)" % (what, kvq_status_string(status), status))
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """The loaded libkvq.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkvq.so is not built (run quantized_decode_attn_amd/build.py "
                              "or __graft_entry__.build()); there is no fallback path")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        L.kvq_status_string.restype = C.c_char_p
        L.kvq_status_string.argtypes = [i32]
        L.kvq_cache_layout.restype = i32
        L.kvq_cache_layout.argtypes = [C.POINTER(KvqConfig), C.POINTER(KvqLayout)]
        L.kvq_paged_layout.restype = i32
        L.kvq_paged_layout.argtypes = [C.POINTER(KvqConfig), i32, C.POINTER(KvqLayout)]
        L.kvq_quantize_append_seqs.restype = i32
        L.kvq_quantize_append_seqs.argtypes = [C.POINTER(KvqCache), vp, vp, i64, C.POINTER(C.c_int64), vp, vp]
        L.kvq_cache_init.restype = i32
        L.kvq_cache_init.argtypes = [C.POINTER(KvqCache), vp]
        L.kvq_quantize_append.restype = i32
        L.kvq_quantize_append.argtypes = [C.POINTER(KvqCache), vp, vp, i64, vp]
        L.kvq_decode_workspace_bytes.restype = C.c_size_t
        L.kvq_decode_workspace_bytes.argtypes = [C.POINTER(KvqCache), i32]
        L.kvq_decode_attention.restype = i32
        L.kvq_decode_attention.argtypes = [C.POINTER(KvqCache), vp, i64, vp, vp, C.c_size_t, i32, vp]
        L.kvq_decode_attention_noalloc.restype = i32
        L.kvq_decode_attention_noalloc.argtypes = [C.POINTER(KvqCache), vp, i64, vp, i32, vp]
        L.kvq_chunk_workspace_bytes.restype = C.c_size_t
        L.kvq_chunk_workspace_bytes.argtypes = [C.POINTER(KvqCache), i32, i32]
        L.kvq_chunk_attention.restype = i32
        L.kvq_chunk_attention.argtypes = [C.POINTER(KvqCache), vp, i32, i64, vp, vp, C.c_size_t, i32, vp]
        L.kvq_decode_step.restype = i32
        L.kvq_decode_step.argtypes = [C.POINTER(KvqCache), vp, vp, vp, vp, vp, C.c_size_t, i32, vp]
        L.kvq_dequantize.restype = i32
        L.kvq_dequantize.argtypes = [C.POINTER(KvqCache), i32, i64, i64, vp, vp]
        _lib = L
    return _lib


# ------------------------------------------------------------------ C ABI, same names
def kvq_status_string(status: int) -> str:
    return lib().kvq_status_string(status).decode()


def kvq_cache_layout(cfg: KvqConfig) -> KvqLayout:
    out = KvqLayout()
    st = lib().kvq_cache_layout(C.byref(cfg), C.byref(out))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_cache_layout")
    return out


def kvq_paged_layout(cfg: KvqConfig, num_blocks: int) -> KvqLayout:
    out = KvqLayout()
    st = lib().kvq_paged_layout(C.byref(cfg), int(num_blocks), C.byref(out))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_paged_layout")
    return out


def kvq_quantize_append_seqs(cache: KvqCache, k_new, v_new, n_max: int, n_host, n_dev, stream=None) -> None:
    """n_host: a ctypes int64 array of the per-sequence counts; n_dev: the same on the
    device (an int64 tensor)."""
    st = lib().kvq_quantize_append_seqs(C.byref(cache), _ptr(k_new), _ptr(v_new), int(n_max),
                                        C.cast(n_host, C.POINTER(C.c_int64)), _ptr(n_dev), _stream(stream))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_quantize_append_seqs")


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def kvq_cache_init(cache: KvqCache, stream=None) -> None:
    st = lib().kvq_cache_init(C.byref(cache), _stream(stream))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_cache_init")


def kvq_quantize_append(cache: KvqCache, k_new, v_new, n_new: int, stream=None) -> None:
    st = lib().kvq_quantize_append(C.byref(cache), _ptr(k_new), _ptr(v_new), int(n_new), _stream(stream))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_quantize_append")


def kvq_decode_workspace_bytes(cache: KvqCache, num_splits: int = 0) -> int:
    return int(lib().kvq_decode_workspace_bytes(C.byref(cache), int(num_splits)))


def kvq_decode_attention(cache: KvqCache, q, q_pos: int, out, ws, ws_bytes: int, num_splits: int = 0,
                         stream=None) -> None:
    st = lib().kvq_decode_attention(C.byref(cache), _ptr(q), int(q_pos), _ptr(out), _ptr(ws),
                                    int(ws_bytes), int(num_splits), _stream(stream))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_decode_attention")


def kvq_decode_attention_noalloc(cache: KvqCache, q, q_pos: int, out, num_splits: int = 0,
                                 stream=None) -> None:
    st = lib().kvq_decode_attention_noalloc(C.byref(cache), _ptr(q), int(q_pos), _ptr(out),
                                            int(num_splits), _stream(stream))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_decode_attention_noalloc")


def kvq_chunk_workspace_bytes(cache: KvqCache, nq: int, num_splits: int = 0) -> int:
    return int(lib().kvq_chunk_workspace_bytes(C.byref(cache), int(nq), int(num_splits)))


def kvq_chunk_attention(cache: KvqCache, q, nq: int, q_pos: int, out, ws, ws_bytes: int, num_splits: int = 0,
                        stream=None) -> None:
    st = lib().kvq_chunk_attention(C.byref(cache), _ptr(q), int(nq), int(q_pos), _ptr(out), _ptr(ws),
                                   int(ws_bytes), int(num_splits), _stream(stream))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_chunk_attention")


def kvq_decode_step(cache: KvqCache, k_new, v_new, q, out, ws, ws_bytes: int, num_splits: int = 0,
                    stream=None) -> None:
    st = lib().kvq_decode_step(C.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), _ptr(ws), ws_bytes,
                               num_splits, _stream(stream))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_decode_step")


def kvq_dequantize(cache: KvqCache, which: int, t0: int, t1: int, out, stream=None) -> None:
    st = lib().kvq_dequantize(C.byref(cache), int(which), int(t0), int(t1), _ptr(out), _stream(stream))
    if st != KVQ_OK:
        raise KvqError(st, "kvq_dequantize")


# ------------------------------------------------------------------ convenience wrapper
_CFG_FIELDS = [f[0] for f in KvqConfig._fields_]


def _check_tensor(t, name: str, shape: tuple, dtype, device) -> None:
    """A tensor handed to the C ABI must have the layout the library reads: the exact
    shape, dtype, contiguous storage and the cache's device."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s is on %s, the cache on %s" % (name, t.device, device))


def make_config(cfg: dict) -> KvqConfig:
    d = dict(cfg)
    d.setdefault("capacity", d.get("tokens"))
    d.setdefault("keep_pct", 0)
    d.setdefault("v_mode", 0)
    return KvqConfig(**{k: d[k] for k in _CFG_FIELDS})


class Cache:
    """Device buffers of one cache (torch uint8 tensors sized by kvq_cache_layout) and the
    C descriptor pointing at them.  ``lut`` (codebook keys) is a uint16 tensor
    ``[kv_heads][D][2**k_bits]`` of fp16 bits, or None; ``vlut`` (codebook values,
    v_mode 1) the same ``[kv_heads][D][2**v_bits]``."""

    def __init__(self, cfg: dict, device="cuda", lut=None, stream=None, vlut=None):
        self.cfg = dict(cfg)
        self.cfg.setdefault("capacity", self.cfg["tokens"])
        self.c_cfg = make_config(self.cfg)
        self.desc = KvqCache()
        self.desc.cfg = self.c_cfg
        self._alloc(kvq_cache_layout(self.c_cfg), device, lut, vlut)
        kvq_cache_init(self.desc, stream)
        self._ws = None

    def _alloc(self, layout, device, lut, vlut=None) -> None:
        import torch
        self.layout = layout
        self.bufs = {}
        for name in BUFFERS:
            size = getattr(self.layout, name)
            if name in ("k_lut", "v_lut"):
                book = lut if name == "k_lut" else vlut
                if size:
                    if book is None:
                        raise ValueError("a codebook is required for %s" % ("k_mode 1" if name == "k_lut" else "v_mode 1"))
                    t = book.to(device=device).contiguous().view(torch.uint8).reshape(-1)
                    if t.numel() != size:
                        raise ValueError("codebook has %d bytes, expected %d" % (t.numel(), size))
                    self.bufs[name] = t
                    setattr(self.desc, name, t.data_ptr())
                continue
            if size:
                t = torch.zeros(size, dtype=torch.uint8, device=device)
                self.bufs[name] = t
                setattr(self.desc, name, t.data_ptr())

    @property
    def length(self) -> int:
        return int(self.desc.length)

    @property
    def device(self):
        return self.bufs["rope"].device

    def append(self, k_new, v_new, stream=None) -> None:
        """k_new, v_new: fp16 tensors [B][Hkv][N][D] on the device (keys pre-RoPE)."""
        import torch
        B, H, D = self.cfg["batch"], self.cfg["kv_heads"], self.cfg["head_dim"]
        if k_new.dim() != 4:
            raise ValueError("k_new must be [B][Hkv][N][D]")
        n = k_new.shape[2]
        _check_tensor(k_new, "k_new", (B, H, n, D), torch.float16, self.device)
        _check_tensor(v_new, "v_new", (B, H, n, D), torch.float16, self.device)
        kvq_quantize_append(self.desc, k_new, v_new, n, stream)

    def workspace(self, num_splits: int = 0):
        import torch
        need = kvq_decode_workspace_bytes(self.desc, num_splits)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 4), dtype=torch.uint8, device=self.bufs["rope"].device)
        return self._ws

    def decode(self, q, q_pos: int | None = None, num_splits: int = 0, out=None, stream=None):
        """q: fp16 [B][Hq][D] on the device (pre-RoPE).  Returns fp32 [B][Hq][D]."""
        import torch
        if q_pos is None:
            q_pos = self.length - 1
        shape = (self.cfg["batch"], self.cfg["q_heads"], self.cfg["head_dim"])
        _check_tensor(q, "q", shape, torch.float16, self.device)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=q.device)
        _check_tensor(out, "out", shape, torch.float32, self.device)
        ws = self.workspace(num_splits)
        kvq_decode_attention(self.desc, q, q_pos, out, ws, ws.numel(), num_splits, stream)
        return out

    def chunk(self, q, q_pos: int | None = None, num_splits: int = 0, out=None, stream=None):
        """q: fp16 [B][Hq][nq][D] on the device (pre-RoPE), queries at positions q_pos ..
        q_pos + nq - 1 (default: the last nq tokens of the cache), each attending
        causally.  Returns fp32 [B][Hq][nq][D]."""
        import torch
        if q.dim() != 4:
            raise ValueError("q must be [B][Hq][nq][D]")
        nq = q.shape[2]
        if q_pos is None:
            q_pos = self.length - nq
        shape = (self.cfg["batch"], self.cfg["q_heads"], nq, self.cfg["head_dim"])
        _check_tensor(q, "q", shape, torch.float16, self.device)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=q.device)
        _check_tensor(out, "out", shape, torch.float32, self.device)
        need = kvq_chunk_workspace_bytes(self.desc, nq, num_splits)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 4), dtype=torch.uint8, device=self.device)
        kvq_chunk_attention(self.desc, q, nq, q_pos, out, self._ws, self._ws.numel(), num_splits, stream)
        return out

    def step(self, k_new, v_new, q, num_splits: int = 0, out=None, stream=None):
        """One fused decode step: append k_new, v_new (fp16 [B][Hkv][D], keys pre-RoPE) and
        attend with q (fp16 [B][Hq][D]) at the new token's position (num_splits 0: the
        library's choice, one launch for a short cache).  Returns fp32 [B][Hq][D]."""
        import torch
        B, H, Hq, D = self.cfg["batch"], self.cfg["kv_heads"], self.cfg["q_heads"], self.cfg["head_dim"]
        _check_tensor(k_new, "k_new", (B, H, D), torch.float16, self.device)
        _check_tensor(v_new, "v_new", (B, H, D), torch.float16, self.device)
        _check_tensor(q, "q", (B, Hq, D), torch.float16, self.device)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        _check_tensor(out, "out", (B, Hq, D), torch.float32, self.device)
        ws = self.workspace(num_splits)
        kvq_decode_step(self.desc, k_new, v_new, q, out, ws, ws.numel(), num_splits, stream)
        return out

    def dequantize(self, which: int, t0: int = 0, t1: int | None = None, stream=None):
        import torch
        if t1 is None:
            t1 = self.length
        B, H, D = self.cfg["batch"], self.cfg["kv_heads"], self.cfg["head_dim"]
        out = torch.empty((B, H, t1 - t0, D), dtype=torch.float32, device=self.bufs["rope"].device)
        kvq_dequantize(self.desc, which, t0, t1, out, stream)
        return out

    def buffer(self, name: str):
        """The raw device buffer (uint8) of one layout entry."""
        return self.bufs.get(name)


class PagedCache(Cache):
    """A cache whose sequences each have their own length.  With ``block_table`` (int32
    ``[batch][capacity / k_block]`` on the device: the physical block of each logical
    block) the quantized blocks live in a pool of ``num_blocks`` physical blocks (the
    paged layout); without it the buffers keep the dense per-sequence slots.  The table
    is read at every call, so the caller may rewrite it in place between calls (a
    serving loop's block allocator); every block a sequence holds or an append completes
    must map to its own physical block."""

    def __init__(self, cfg: dict, num_blocks: int | None = None, block_table=None, device="cuda", lut=None,
                 stream=None, vlut=None):
        import torch
        self.cfg = dict(cfg)
        self.cfg.setdefault("capacity", self.cfg["tokens"])
        self.c_cfg = make_config(self.cfg)
        self.desc = KvqCache()
        self.desc.cfg = self.c_cfg
        B = self.cfg["batch"]
        if block_table is not None:
            nb = self.cfg["capacity"] // self.cfg["k_block"]
            _check_tensor(block_table, "block_table", (B, nb), torch.int32, torch.device(device))
            if num_blocks is None:
                raise ValueError("a block table needs num_blocks")
            layout = kvq_paged_layout(self.c_cfg, num_blocks)
            self.block_table = block_table
            self.desc.block_table = block_table.data_ptr()
            self.desc.num_blocks = int(num_blocks)
        else:
            layout = kvq_cache_layout(self.c_cfg)
            self.block_table = None
        self._alloc(layout, device, lut, vlut)
        self.seq_lens_dev = torch.zeros(B, dtype=torch.int64, device=device)
        self._seq_lens_host = (C.c_int64 * B)()
        self.desc.seq_lens = self.seq_lens_dev.data_ptr()
        self.desc.seq_lens_host = C.cast(self._seq_lens_host, C.POINTER(C.c_int64))
        kvq_cache_init(self.desc, stream)
        self._ws = None

    @property
    def lengths(self) -> list:
        return [int(x) for x in self._seq_lens_host]

    @property
    def length(self) -> int:
        raise AttributeError("a PagedCache has one length per sequence: use .lengths")

    def append_seqs(self, k_new, v_new, counts, stream=None) -> None:
        """Sequence b takes the first counts[b] rows of k_new[b], v_new[b] (fp16
        [B][Hkv][n_max][D] on the device, keys pre-RoPE)."""
        import torch
        B, H, D = self.cfg["batch"], self.cfg["kv_heads"], self.cfg["head_dim"]
        if k_new.dim() != 4:
            raise ValueError("k_new must be [B][Hkv][n_max][D]")
        n_max = k_new.shape[2]
        _check_tensor(k_new, "k_new", (B, H, n_max, D), torch.float16, self.device)
        _check_tensor(v_new, "v_new", (B, H, n_max, D), torch.float16, self.device)
        counts = [int(x) for x in counts]
        if len(counts) != B:
            raise ValueError("one count per sequence")
        n_host = (C.c_int64 * B)(*counts)
        n_dev = torch.tensor(counts, dtype=torch.int64, device=self.device)
        kvq_quantize_append_seqs(self.desc, k_new, v_new, n_max, n_host, n_dev, stream)
        self._last_counts = n_dev   # kept alive until the stream has read it

    def decode(self, q, num_splits: int = 0, out=None, stream=None):
        """Every sequence's query (fp16 [B][Hq][D], pre-RoPE) at its own newest token.
        Returns fp32 [B][Hq][D]."""
        import torch
        shape = (self.cfg["batch"], self.cfg["q_heads"], self.cfg["head_dim"])
        _check_tensor(q, "q", shape, torch.float16, self.device)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=q.device)
        _check_tensor(out, "out", shape, torch.float32, self.device)
        ws = self.workspace(num_splits)
        kvq_decode_attention(self.desc, q, -1, out, ws, ws.numel(), num_splits, stream)
        return out
