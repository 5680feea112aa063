"""Host-side checks of the C ABI: the library loads, exports every entry point that
include/kvq.h declares, sizes buffers like the layout the oracle implements, and
rejects bad arguments before touching a GPU.  No kernel runs here."""
import ctypes as C
import os
import re

import pytest

import quantized_decode_attn_amd as kvq
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kvq.LIB_PATH):
        import quantized_decode_attn_amd.build as b
        b.build()
    return kvq.lib()


def test_exports_every_declared_function(L):
    decl = _declared_functions()
    assert set(decl) == set(kvq.EXPORTED)
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5):
        assert kvq.kvq_status_string(st)
    assert kvq.kvq_status_string(-99) == "unknown status"


VARIANTS = {
    "c1_keep5": dict(keep_pct=5),
    "c3_vlut": dict(v_mode=1),
    "c0_vlut2": dict(v_mode=1, v_bits=2, v_group=32),
    "c1_fp8": dict(k_mode=2, k_bits=8, v_mode=2, v_bits=8),
}


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4", "c1_keep5", "c3_vlut", "c0_vlut2", "c1_fp8"])
def test_layout_matches_oracle_layout(L, orc, name):
    cfg = synth.config(name[:2], **VARIANTS.get(name, {}))
    lay = kvq.kvq_cache_layout(kvq.make_config(cfg))
    ref = orc.layout(cfg)
    for k, v in ref.items():
        assert getattr(lay, k) == v, k
    D = cfg["head_dim"]
    assert lay.rope == (cfg["k_block"] + cfg["tokens"] // cfg["k_block"]) * D * 4


def _status(cfg):
    return L_layout(kvq.make_config(cfg))


def L_layout(c):
    out = kvq.KvqLayout()
    return kvq.lib().kvq_cache_layout(C.byref(c), C.byref(out))


@pytest.mark.parametrize("field,value,want", [
    ("head_dim", 0, kvq.KVQ_EINVAL), ("head_dim", 63, kvq.KVQ_EINVAL), ("head_dim", 96, kvq.KVQ_EINVAL),
    ("head_dim", 256, kvq.KVQ_EUNSUPPORTED),
    ("k_bits", 0, kvq.KVQ_EINVAL), ("k_bits", 5, kvq.KVQ_EUNSUPPORTED), ("v_bits", 3, kvq.KVQ_EUNSUPPORTED),
    ("v_group", 48, kvq.KVQ_EINVAL), ("v_group", 8, kvq.KVQ_EUNSUPPORTED), ("k_block", 100, kvq.KVQ_EINVAL),
    ("k_block", 32, kvq.KVQ_EUNSUPPORTED), ("q_heads", 6, kvq.KVQ_EINVAL), ("clip_quantile", 1.0, kvq.KVQ_EINVAL),
    ("clip_quantile", -0.1, kvq.KVQ_EINVAL), ("outlier_pct", 101, kvq.KVQ_EINVAL), ("outlier_pct", 4, kvq.KVQ_EUNSUPPORTED),
    ("rope_theta", 0.5, kvq.KVQ_EINVAL), ("k_mode", 3, kvq.KVQ_EINVAL), ("capacity", 0, kvq.KVQ_EINVAL),
    ("v_mode", 3, kvq.KVQ_EINVAL), ("v_mode", -1, kvq.KVQ_EINVAL),
    ("k_mode", 2, kvq.KVQ_EINVAL), ("v_mode", 2, kvq.KVQ_EINVAL),              # FP8 needs both, 8 bits
])
def test_layout_rejects(L, field, value, want):
    cfg = synth.config("c1", q_heads=32, kv_heads=8)
    cfg[field] = value
    assert _status(cfg) == want


def test_value_codebook_excludes_outliers_and_clipping(L):
    """Codebook values replace the uniform value range that outliers and clipping act
    on: either with v_mode 1 is refused; keys kept in fp16 combine with it."""
    assert _status(synth.config("c1", v_mode=1)) == kvq.KVQ_OK
    assert _status(synth.config("c2", v_mode=1)) == kvq.KVQ_EUNSUPPORTED          # 1% outliers
    assert _status(synth.config("c4", v_mode=1)) == kvq.KVQ_EUNSUPPORTED          # clip + outliers
    assert _status(synth.config("c1", v_mode=1, keep_pct=5)) == kvq.KVQ_OK


def _fake_cache(cfg, length=0):
    """A descriptor whose buffer pointers are non-null but never dereferenced (only
    paths that fail before enqueueing anything are exercised)."""
    c = kvq.KvqCache()
    c.cfg = kvq.make_config(cfg)
    lay = kvq.kvq_cache_layout(c.cfg)
    for n in kvq.BUFFERS:
        if getattr(lay, n):
            setattr(c, n, 0x1000)
    c.length = length
    return c


def test_append_errors_leave_cache_unchanged(L):
    cfg = synth.config("c0")
    c = _fake_cache(cfg, length=200)
    assert L.kvq_quantize_append(C.byref(c), 0x1000, 0x1000, 57, None) == kvq.KVQ_ECAPACITY
    assert c.length == 200
    assert L.kvq_quantize_append(C.byref(c), 0x1000, 0x1000, -1, None) == kvq.KVQ_EINVAL
    assert L.kvq_quantize_append(C.byref(c), None, 0x1000, 8, None) == kvq.KVQ_EINVAL
    assert L.kvq_quantize_append(C.byref(c), 0x1000, 0x1000, 0, None) == kvq.KVQ_OK
    assert c.length == 200
    c.v_scale = None
    assert L.kvq_quantize_append(C.byref(c), 0x1000, 0x1000, 8, None) == kvq.KVQ_EINVAL
    c2 = _fake_cache(synth.config("c2"), length=5)
    c2.k_col = None                                            # outliers on: CSR buffers required
    assert L.kvq_quantize_append(C.byref(c2), 0x1000, 0x1000, 8, None) == kvq.KVQ_EINVAL
    c3 = _fake_cache(synth.config("c3"))
    c3.k_lut = None                                            # codebook keys need the codebook
    assert L.kvq_quantize_append(C.byref(c3), 0x1000, 0x1000, 8, None) == kvq.KVQ_EINVAL
    assert c3.length == 0


def test_decode_and_dequantize_argument_errors(L):
    cfg = synth.config("c0")
    c = _fake_cache(cfg, length=0)
    ws = L.kvq_decode_workspace_bytes(C.byref(c), 4)
    assert ws == 1 * 4 * 4 * (64 + 2) * 4
    assert L.kvq_decode_attention(C.byref(c), 0x1000, 0, 0x1000, 0x1000, ws, 4, None) == kvq.KVQ_EINVAL
    c.length = 100
    assert L.kvq_decode_attention(C.byref(c), 0x1000, 99, 0x1000, 0x1000, ws - 4, 4, None) == kvq.KVQ_EWORKSPACE
    assert L.kvq_decode_attention(C.byref(c), 0x1000, -1, 0x1000, 0x1000, ws, 4, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attention(C.byref(c), None, 99, 0x1000, 0x1000, ws, 4, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attention(C.byref(c), 0x1000, 99, 0x1000, None, ws, 4, None) == kvq.KVQ_EWORKSPACE
    big = L.kvq_decode_workspace_bytes(C.byref(c), 4097)
    assert L.kvq_decode_attention(C.byref(c), 0x1000, 99, 0x1000, 0x1000, big, 4097, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attention(C.byref(c), 0x1000, 99, 0x1000, 0x1000, big, -2, None) == kvq.KVQ_EINVAL
    assert L.kvq_dequantize(C.byref(c), 2, 0, 10, 0x1000, None) == kvq.KVQ_EINVAL
    assert L.kvq_dequantize(C.byref(c), 0, 5, 4, 0x1000, None) == kvq.KVQ_EINVAL
    assert L.kvq_dequantize(C.byref(c), 0, 0, 101, 0x1000, None) == kvq.KVQ_EINVAL
    assert L.kvq_dequantize(C.byref(c), 1, 7, 7, None, None) == kvq.KVQ_OK
    assert L.kvq_decode_workspace_bytes(None, 4) == 0
