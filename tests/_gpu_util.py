"""Helpers of the GPU parity tests: build a cache through the C ABI from the seeded
inputs, build the same heads with the CPU oracle, and compare buffers bit for bit
over the regions the layout defines."""
from __future__ import annotations

import sys

import numpy as np

import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def keep_count(cfg: dict) -> int:
    p = cfg.get("keep_pct", 0)
    return (p * cfg["k_block"] + 99) // 100 if p > 0 else 0


def per_head_bytes(cfg: dict, ko: int) -> dict:
    D, T, Bk = cfg["head_dim"], cfg["capacity"], cfg["k_block"]
    ng = D // cfg["v_group"]
    uni = cfg["k_mode"] == 0
    vuni = cfg.get("v_mode", 0) == 0
    R = keep_count(cfg)
    return {
        "k_keep_idx": (T // Bk) * R,
        "k_keep_val": (T // Bk) * R * D * 2,
        "k_codes": T * D * cfg["k_bits"] // 8,
        "k_scale": (T // Bk) * D * 2 if uni else 0,
        "k_zero": (T // Bk) * D * 2 if uni else 0,
        "k_tail": Bk * D * 2,
        "v_codes": T * D * cfg["v_bits"] // 8,
        "v_scale": T * ng * 2 if vuni else 0,
        "v_zero": T * ng * 2 if vuni else 0,
        "v_tail": Bk * D * 2,
        "k_rowptr": (T + 1) * 4 if ko else 0,
        "k_col": T * ko,
        "k_val": T * ko * 2,
        "v_rowptr": (T + 1) * 4 if ko else 0,
        "v_col": T * ko,
        "v_val": T * ko * 2,
    }


def defined_bytes(cfg: dict, ko: int, length: int) -> dict:
    """Number of leading bytes of each per-head buffer that a cache of `length`
    tokens defines."""
    D, Bk = cfg["head_dim"], cfg["k_block"]
    nq = (length // Bk) * Bk
    nt = length - nq
    ng = D // cfg["v_group"]
    uni = cfg["k_mode"] == 0
    vuni = cfg.get("v_mode", 0) == 0
    R = keep_count(cfg)
    return {
        "k_keep_idx": (nq // Bk) * R,
        "k_keep_val": (nq // Bk) * R * D * 2,
        "k_codes": nq * D * cfg["k_bits"] // 8,
        "k_scale": (nq // Bk) * D * 2 if uni else 0,
        "k_zero": (nq // Bk) * D * 2 if uni else 0,
        "k_tail": nt * D * 2,
        "v_codes": nq * D * cfg["v_bits"] // 8,
        "v_scale": nq * ng * 2 if vuni else 0,
        "v_zero": nq * ng * 2 if vuni else 0,
        "v_tail": nt * D * 2,
        "k_rowptr": (nq + 1) * 4 if ko and nq else 0,
        "k_col": nq * ko,
        "k_val": nq * ko * 2,
        "v_rowptr": (nq + 1) * 4 if ko and nq else 0,
        "v_col": nq * ko,
        "v_val": nq * ko * 2,
    }


def gpu_head_bytes(cache, name: str, bh: int, per: int, nbytes: int) -> np.ndarray:
    buf = cache.buffer(name)
    return buf[bh * per: bh * per + nbytes].cpu().numpy()


def oracle_head_bytes(hc, name: str, nbytes: int) -> np.ndarray:
    return np.ascontiguousarray(getattr(hc, name)).view(np.uint8).reshape(-1)[:nbytes]


def compare_head(cache, hc, cfg: dict, ko: int, b: int, h: int) -> None:
    bh = b * cfg["kv_heads"] + h
    per = per_head_bytes(cfg, ko)
    need = defined_bytes(cfg, ko, hc.length)
    for name, nb in need.items():
        if nb == 0:
            continue
        g = gpu_head_bytes(cache, name, bh, per[name], nb)
        o = oracle_head_bytes(hc, name, nb)
        if not np.array_equal(g, o):
            bad = np.nonzero(g != o)[0]
            raise AssertionError("%s differs at (b=%d, h=%d): %d of %d bytes, first at byte %d "
                                 "(gpu %d, oracle %d)" % (name, b, h, bad.size, nb, bad[0], g[bad[0]], o[bad[0]]))


def upload(x: np.ndarray):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.float16)


def build_gpu_cache(cfg: dict, k: np.ndarray, v: np.ndarray, chunks=None, lut=None, vlut=None):
    """A library cache filled with ``k``/``v`` (fp16 bits [B][Hkv][T][D]) through
    kvq_quantize_append, in one call or in the given chunk sizes."""
    import quantized_decode_attn_amd as kvq
    torch, dev = torch_dev()
    lut_t = None if lut is None else torch.from_numpy(lut.view(np.int16)).to(dev)
    vlut_t = None if vlut is None else torch.from_numpy(vlut.view(np.int16)).to(dev)
    cache = kvq.Cache(cfg, device=dev, lut=lut_t, vlut=vlut_t)
    T = k.shape[2]
    chunks = chunks or [T]
    assert sum(chunks) == T
    t = 0
    for n in chunks:
        if n:
            cache.append(upload(k[:, :, t:t + n]), upload(v[:, :, t:t + n]))
        t += n
    torch.cuda.synchronize()
    return cache


def oracle_heads(cfg: dict, k: np.ndarray, v: np.ndarray, lut=None, heads=None, vlut=None) -> dict:
    import oracle
    out = {}
    B, H = k.shape[0], k.shape[1]
    for b in range(B):
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                continue
            hc = oracle.HeadCache(cfg, None if lut is None else lut[h], None if vlut is None else vlut[h])
            hc.build(k[b, h], v[b, h])
            out[(b, h)] = hc
    return out


def inputs(cfg: dict, t0: int = 0, t1: int | None = None):
    k = synth.gen_tensor(cfg, synth.TENSOR_K, t0, t1)
    v = synth.gen_tensor(cfg, synth.TENSOR_V, t0, t1)
    return k, v
