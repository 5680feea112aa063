"""CPU oracle for low-bit KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; the product path never touches
it.  The arithmetic lives in ``oracle.c`` (plain scalar C, fp32 quantizer with
every operation rounded separately, fp64 attention); this module only compiles
it with gcc and marshals numpy arrays.  It shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "_build", "liborc.so")


GCC_FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
             "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def compile_source(src: str, out: str) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``oracle/_build/liborc.so`` with gcc."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


class Cfg(C.Structure):
    _fields_ = [("batch", C.c_int32), ("q_heads", C.c_int32), ("kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("capacity", C.c_int32), ("k_bits", C.c_int32),
                ("k_mode", C.c_int32), ("k_block", C.c_int32), ("v_bits", C.c_int32),
                ("v_group", C.c_int32), ("clip_quantile", C.c_float), ("outlier_pct", C.c_int32),
                ("rope_theta", C.c_float), ("keep_pct", C.c_int32), ("v_mode", C.c_int32)]


class _Head(C.Structure):
    _fields_ = [("k_codes", C.c_void_p), ("k_scale", C.c_void_p), ("k_zero", C.c_void_p),
                ("k_lut", C.c_void_p), ("k_tail", C.c_void_p), ("v_codes", C.c_void_p),
                ("v_scale", C.c_void_p), ("v_zero", C.c_void_p), ("v_tail", C.c_void_p),
                ("k_rowptr", C.c_void_p), ("k_col", C.c_void_p), ("k_val", C.c_void_p),
                ("v_rowptr", C.c_void_p), ("v_col", C.c_void_p), ("v_val", C.c_void_p),
                ("k_keep_idx", C.c_void_p), ("k_keep_val", C.c_void_p), ("v_lut", C.c_void_p),
                ("length", C.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = load(_LIB if os.path.exists(_LIB) else build())
    return _lib


def use_library(path: str | None):
    """Point this module at another build of ``oracle.c`` (used by the planted-mistake
    tests); ``None`` returns to the default build."""
    global _lib
    _lib = None if path is None else load(path)


def load(path: str):
    """Open one build of ``oracle.c`` and declare its entry points."""
    L = C.CDLL(path)
    vp, i64 = C.c_void_p, C.c_int64
    sig = {
        "orc_h2f": (C.c_float, [C.c_uint16]),
        "orc_f2h_rn": (C.c_uint16, [C.c_float]),
        "orc_h2f_array": (None, [vp, vp, i64]),
        "orc_f2h_array": (None, [vp, vp, i64, C.c_int]),
        "orc_kv_bytes": (C.c_double, [i64, i64, i64, i64, i64]),
        "orc_kout": (C.c_int, [C.POINTER(Cfg)]),
        "orc_f_to_e4m3": (C.c_uint8, [C.c_uint16]),
        "orc_e4m3_to_f": (C.c_float, [C.c_uint8]),
        "orc_keep_count": (C.c_int, [C.POINTER(Cfg)]),
        "orc_layout": (None, [C.POINTER(Cfg), vp]),
        "orc_clip_threshold": (C.c_float, [vp, i64, C.c_float]),
        "orc_quantize_block": (C.c_int, [C.POINTER(Cfg), C.c_int, i64, vp, C.POINTER(_Head)]),
        "orc_build_head": (C.c_int, [C.POINTER(Cfg), C.POINTER(_Head), vp, vp, i64]),
        "orc_build_heads": (C.c_int, [C.POINTER(Cfg), i64, vp, vp, vp, i64]),
        "orc_dequantize_head": (C.c_int, [C.POINTER(Cfg), C.POINTER(_Head), C.c_int, i64, i64, vp]),
        "orc_decode_head": (C.c_int, [C.POINTER(Cfg), C.POINTER(_Head), vp, i64, vp]),
        "orc_decode_many": (C.c_int, [C.POINTER(Cfg), i64, vp, vp, vp, vp]),
        "orc_chunk_head": (C.c_int, [C.POINTER(Cfg), C.POINTER(_Head), vp, C.c_int32, i64, vp]),
        "orc_chunk_many": (C.c_int, [C.POINTER(Cfg), i64, vp, vp, C.c_int32, vp, vp]),
        "orc_max_threads": (C.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


LAYOUT_NAMES = ["k_codes", "k_scale", "k_zero", "k_lut", "k_tail", "v_codes", "v_scale",
                "v_zero", "v_tail", "k_rowptr", "k_col", "k_val", "v_rowptr", "v_col", "v_val",
                "k_keep_idx", "k_keep_val", "v_lut"]

_CFG_KEYS = [f[0] for f in Cfg._fields_]


def make_cfg(cfg: dict) -> Cfg:
    """A C configuration from a workload dict (``synth.CONFIGS`` style); ``capacity``
    defaults to ``tokens``."""
    d = dict(cfg)
    d.setdefault("capacity", d.get("tokens"))
    d.setdefault("keep_pct", 0)
    d.setdefault("v_mode", 0)
    return Cfg(**{k: d[k] for k in _CFG_KEYS})


def kout(cfg: dict) -> int:
    c = make_cfg(cfg)
    return lib().orc_kout(C.byref(c))


def keep_count(cfg: dict) -> int:
    """Key vectors kept in fp16 per quantized block."""
    c = make_cfg(cfg)
    return lib().orc_keep_count(C.byref(c))


def layout(cfg: dict) -> dict:
    c = make_cfg(cfg)
    out = np.zeros(18, np.int64)
    lib().orc_layout(C.byref(c), out.ctypes.data)
    return dict(zip(LAYOUT_NAMES, (int(v) for v in out)))


def e4m3_from_f16(bits) -> np.ndarray:
    """fp16 bits -> OCP E4M3 bytes (nearest, ties to even, saturating to +-448)."""
    b = np.asarray(bits, np.uint16).reshape(-1)
    L = lib()
    return np.array([L.orc_f_to_e4m3(int(x)) for x in b], np.uint8).reshape(np.shape(bits))


def e4m3_to_f(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8).reshape(-1)
    L = lib()
    return np.array([L.orc_e4m3_to_f(int(x)) for x in c], np.float32).reshape(np.shape(codes))


def h2f(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16)
    f = np.empty(h.shape, np.float32)
    lib().orc_h2f_array(h.ctypes.data, f.ctypes.data, h.size)
    return f


def f2h(f: np.ndarray, mode: str = "rn") -> np.ndarray:
    f = np.ascontiguousarray(f, np.float32)
    h = np.empty(f.shape, np.uint16)
    lib().orc_f2h_array(f.ctypes.data, h.ctypes.data, f.size, {"rn": 0, "rd": 1, "ru": 2}[mode])
    return h


def kv_bytes(layers, batch, tokens, hidden, bits) -> float:
    return lib().orc_kv_bytes(layers, batch, tokens, hidden, bits)


def clip_threshold(block_bits: np.ndarray, q: float) -> float:
    b = np.ascontiguousarray(block_bits, np.uint16)
    return float(lib().orc_clip_threshold(b.ctypes.data, b.size, q))


class HeadCache:
    """Host buffers of one (batch, kv-head) of the quantized cache, in the library's
    per-(b, h) layout."""

    def __init__(self, cfg: dict, lut_head: np.ndarray | None = None, vlut_head: np.ndarray | None = None):
        self.cfg = dict(cfg)
        self.cfg.setdefault("capacity", self.cfg["tokens"])
        c = self.cfg
        D, T, Bk = c["head_dim"], c["capacity"], c["k_block"]
        ko = kout(c)
        self.kout = ko
        uni = c["k_mode"] == 0
        self.k_codes = np.zeros(T * D * c["k_bits"] // 8, np.uint8)
        self.k_scale = np.zeros((T // Bk, D) if uni else (0,), np.uint16)
        self.k_zero = np.zeros((T // Bk, D) if uni else (0,), np.uint16)
        if c["k_mode"] == 1:
            assert lut_head is not None and lut_head.shape == (D, 1 << c["k_bits"])
            self.k_lut = np.ascontiguousarray(lut_head, np.uint16)
        else:
            self.k_lut = np.zeros(0, np.uint16)
        self.k_tail = np.zeros((Bk, D), np.uint16)
        self.v_codes = np.zeros(T * D * c["v_bits"] // 8, np.uint8)
        ng = D // c["v_group"]
        vuni = c.get("v_mode", 0) == 0
        self.v_scale = np.zeros((T, ng) if vuni else (0,), np.uint16)
        self.v_zero = np.zeros((T, ng) if vuni else (0,), np.uint16)
        if c.get("v_mode", 0) == 1:
            assert vlut_head is not None and vlut_head.shape == (D, 1 << c["v_bits"])
            self.v_lut = np.ascontiguousarray(vlut_head, np.uint16)
        else:
            self.v_lut = np.zeros(0, np.uint16)
        self.v_tail = np.zeros((Bk, D), np.uint16)
        n = T + 1 if ko else 0
        self.k_rowptr = np.zeros(n, np.int32)
        self.v_rowptr = np.zeros(n, np.int32)
        self.k_col = np.zeros(T * ko, np.uint8)
        self.v_col = np.zeros(T * ko, np.uint8)
        self.k_val = np.zeros(T * ko, np.uint16)
        self.v_val = np.zeros(T * ko, np.uint16)
        R = keep_count(c)
        self.k_keep_idx = np.zeros(T // Bk * R, np.uint8)
        self.k_keep_val = np.zeros((T // Bk * R, D), np.uint16)
        self.length = 0
        self._c = make_cfg(self.cfg)

    def _struct(self) -> _Head:
        s = _Head()
        for f, _ in _Head._fields_:
            if f != "length":
                setattr(s, f, getattr(self, f).ctypes.data)
        s.length = self.length
        return s

    def build(self, k_src: np.ndarray, v_src: np.ndarray) -> "HeadCache":
        """Quantize ``T`` tokens (fp16 bits ``[T][D]``) into this empty head."""
        k = np.ascontiguousarray(k_src, np.uint16)
        v = np.ascontiguousarray(v_src, np.uint16)
        assert k.shape == v.shape and k.shape[1] == self.cfg["head_dim"]
        s = self._struct()
        if lib().orc_build_head(C.byref(self._c), C.byref(s), k.ctypes.data, v.ctypes.data, k.shape[0]):
            raise RuntimeError("oracle build failed")
        self.length = int(s.length)
        return self

    def quantize_block(self, is_key: bool, n: int, src: np.ndarray) -> None:
        src = np.ascontiguousarray(src, np.uint16)
        s = self._struct()
        if lib().orc_quantize_block(C.byref(self._c), int(is_key), n, src.ctypes.data, C.byref(s)):
            raise RuntimeError("oracle quantize failed")

    def dequantize(self, which: int, t0: int = 0, t1: int | None = None) -> np.ndarray:
        if t1 is None:
            t1 = self.length
        out = np.empty((t1 - t0, self.cfg["head_dim"]), np.float32)
        s = self._struct()
        if lib().orc_dequantize_head(C.byref(self._c), C.byref(s), which, t0, t1, out.ctypes.data):
            raise RuntimeError("oracle dequantize: bad range")
        return out

    def decode(self, q_bits: np.ndarray, q_pos: int | None = None) -> np.ndarray:
        """fp64 attention output ``[D]`` of one query (fp16 bits ``[D]``)."""
        if q_pos is None:
            q_pos = self.length - 1
        q = np.ascontiguousarray(q_bits, np.uint16)
        out = np.empty(self.cfg["head_dim"], np.float64)
        s = self._struct()
        if lib().orc_decode_head(C.byref(self._c), C.byref(s), q.ctypes.data, q_pos, out.ctypes.data):
            raise RuntimeError("oracle decode failed")
        return out

    def chunk(self, q_bits: np.ndarray, q_pos: int) -> np.ndarray:
        """fp64 outputs ``[nq][D]`` of ``nq`` consecutive queries (fp16 bits ``[nq][D]``)
        at positions ``q_pos ..``, each attending causally to the cache."""
        q = np.ascontiguousarray(q_bits, np.uint16).reshape(-1, self.cfg["head_dim"])
        out = np.empty(q.shape, np.float64)
        s = self._struct()
        if lib().orc_chunk_head(C.byref(self._c), C.byref(s), q.ctypes.data, q.shape[0], int(q_pos),
                                out.ctypes.data):
            raise RuntimeError("oracle chunk attention failed")
        return out


def decode_many(cfg: dict, heads: list, qs: np.ndarray, q_pos) -> np.ndarray:
    """fp64 outputs ``[n][D]`` for ``n`` (HeadCache, query) pairs, OpenMP across pairs."""
    n = len(heads)
    structs = [h._struct() for h in heads]
    arr = (C.POINTER(_Head) * n)(*[C.pointer(s) for s in structs])
    qs = np.ascontiguousarray(qs, np.uint16).reshape(n, -1)
    pos = np.ascontiguousarray(np.broadcast_to(np.asarray(q_pos, np.int64), (n,)))
    out = np.empty((n, cfg["head_dim"]), np.float64)
    c = make_cfg(cfg)
    if lib().orc_decode_many(C.byref(c), n, C.cast(arr, C.c_void_p), qs.ctypes.data,
                             pos.ctypes.data, out.ctypes.data):
        raise RuntimeError("oracle decode failed")
    return out


def chunk_many(cfg: dict, heads: list, qs: np.ndarray, nq: int, q_pos) -> np.ndarray:
    """fp64 outputs ``[n][nq][D]`` for ``n`` (HeadCache, query chunk) pairs; chunk ``i``
    is ``qs[i]`` (fp16 bits ``[nq][D]``) at positions ``q_pos[i] ..``.  OpenMP across pairs."""
    n = len(heads)
    structs = [h._struct() for h in heads]
    arr = (C.POINTER(_Head) * n)(*[C.pointer(s) for s in structs])
    qs = np.ascontiguousarray(qs, np.uint16).reshape(n, nq, -1)
    pos = np.ascontiguousarray(np.broadcast_to(np.asarray(q_pos, np.int64), (n,)))
    out = np.empty((n, nq, cfg["head_dim"]), np.float64)
    c = make_cfg(cfg)
    if lib().orc_chunk_many(C.byref(c), n, C.cast(arr, C.c_void_p), qs.ctypes.data, int(nq),
                            pos.ctypes.data, out.ctypes.data):
        raise RuntimeError("oracle chunk attention failed")
    return out


def build_heads(cfg: dict, k_src: np.ndarray, v_src: np.ndarray, luts=None, vluts=None) -> list:
    """Quantize ``n`` heads at once (fp16 bits ``[n][T][D]`` each), OpenMP across heads;
    ``luts`` / ``vluts`` give each head's key / value codebook (codebook modes only).
    Returns the HeadCaches."""
    k = np.ascontiguousarray(k_src, np.uint16)
    v = np.ascontiguousarray(v_src, np.uint16)
    n, T = k.shape[0], k.shape[1]
    heads = [HeadCache(cfg, None if luts is None else luts[i], None if vluts is None else vluts[i])
             for i in range(n)]
    arr = (_Head * n)(*[h._struct() for h in heads])
    c = make_cfg(cfg)
    if lib().orc_build_heads(C.byref(c), n, C.cast(arr, C.c_void_p), k.ctypes.data, v.ctypes.data, T):
        raise RuntimeError("oracle build failed")
    for i, h in enumerate(heads):
        h.length = int(arr[i].length)
    return heads


def max_threads() -> int:
    return int(lib().orc_max_threads())


def build_cache(cfg: dict, k_src: np.ndarray, v_src: np.ndarray, lut: np.ndarray | None = None,
                vlut: np.ndarray | None = None) -> list:
    """Quantize whole ``[B][Hkv][T][D]`` sources; returns ``[B][Hkv]`` nested lists of HeadCache."""
    B, H = cfg["batch"], cfg["kv_heads"]
    out = []
    for b in range(B):
        row = []
        for h in range(H):
            hc = HeadCache(cfg, None if lut is None else lut[h], None if vlut is None else vlut[h])
            hc.build(k_src[b, h], v_src[b, h])
            row.append(hc)
        out.append(row)
    return out
