"""Seeded synthetic inputs shaped like the workloads of the low-bit KV-cache pages.

This module draws random numbers and nothing else: it holds none of the
quantization, packing or attention arithmetic.  Both the CPU oracle and the HIP
library are fed from here; neither side imports the other.

Recipe (every draw in float64, then rounded to fp16 with round-to-nearest-even):

* stream ``[seed, 3, h]``: per-channel key std ``LogNormal(0, 0.5)`` for head
  ``h``; two distinct channels of the head are picked from the same stream and
  multiplied by 20 (the strong per-channel outliers that motivate per-channel
  Key quantization in "【LLM量化技术介绍-3】KV Cache量化技术介绍",
  section "Per-Channel Key Quantization").
* stream ``[seed, tensor, b, h, chunk]`` with ``tensor`` 0 (K) or 1 (V) and
  ``chunk = t // 65536``: standard normals for the tokens of that chunk.
  K = N(0,1) * std[h, d] (pre-RoPE), V = N(0,1).
* stream ``[seed, 2, b]``: the decode queries, N(0,1), ``[Hq][D]`` per sequence.
* stream ``[seed, 4, b, h, chunk, tensor]`` (heavy-tail injection, only where a
  workload asks for it): each element is independently replaced with
  probability 0.01 by ``clip(10 * t_3, -200, 200)`` times its channel std (K)
  or times 1 (V).
* stream ``[1, 5, h]``: 4096 calibration key tokens per head for the
  per-channel codebook, fitted by 1-D Lloyd k-means in float64 (input
  preparation only: the codebook is an input of both sides).
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as _mp

import numpy as np

CHUNK = 65536
TENSOR_K, TENSOR_V, TENSOR_Q, TENSOR_STD, TENSOR_INJECT, TENSOR_CALIB, TENSOR_QCHUNK = 0, 1, 2, 3, 4, 5, 6
TENSOR_VCALIB = 7

# The five workloads.  ``tokens`` is the cache length the decode attends over;
# ``existing`` (only the prefill-append workload) is the part already in the
# cache before the timed append.
CONFIGS = {
    "c0": dict(workload="tiny-mha-d64-t256", batch=1, q_heads=4, kv_heads=4, head_dim=64,
               tokens=256, existing=0, k_bits=4, k_mode=0, k_block=64, v_bits=4, v_group=64,
               clip_quantile=0.0, outlier_pct=0, inject=False, rope_theta=10000.0),
    "c1": dict(workload="llama2-7b-layer-b8-h32-d128-t32768-int4", batch=8, q_heads=32,
               kv_heads=32, head_dim=128, tokens=32768, existing=0, k_bits=4, k_mode=0,
               k_block=128, v_bits=4, v_group=128, clip_quantile=0.0, outlier_pct=0,
               inject=False, rope_theta=10000.0),
    "c2": dict(workload="llama3-8b-layer-gqa-b4-hq32-hkv8-t131072-int4-csr1", batch=4,
               q_heads=32, kv_heads=8, head_dim=128, tokens=131072, existing=0, k_bits=4,
               k_mode=0, k_block=128, v_bits=4, v_group=128, clip_quantile=0.0,
               outlier_pct=1, inject=True, rope_theta=10000.0),
    "c3": dict(workload="long-ctx-b1-h32-t1048576-k3lut-v2", batch=1, q_heads=32, kv_heads=32,
               head_dim=128, tokens=1048576, existing=0, k_bits=3, k_mode=1, k_block=128,
               v_bits=2, v_group=64, clip_quantile=0.0, outlier_pct=0, inject=False,
               rope_theta=10000.0),
    "c4": dict(workload="prefill-append-b16-h32-16384on16384-clip99-csr1", batch=16, q_heads=32,
               kv_heads=32, head_dim=128, tokens=32768, existing=16384, k_bits=4, k_mode=0,
               k_block=128, v_bits=4, v_group=128, clip_quantile=0.99, outlier_pct=1,
               inject=False, rope_theta=10000.0),
}


def config(name: str, **overrides) -> dict:
    """A copy of a named workload, optionally with fields replaced (for shrunken test cases)."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    cfg.setdefault("capacity", cfg["tokens"])
    return cfg


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def chan_std(cfg: dict, seed: int = 0) -> np.ndarray:
    """Per-(kv-head, channel) key standard deviations, float64 ``[Hkv][D]``."""
    D = cfg["head_dim"]
    out = np.empty((cfg["kv_heads"], D), np.float64)
    for h in range(cfg["kv_heads"]):
        r = _rng(seed, TENSOR_STD, h)
        s = r.lognormal(0.0, 0.5, D)
        idx = r.choice(D, 2, replace=False)
        s[idx] *= 20.0
        out[h] = s
    return out


def _chunk_rows(cfg: dict, chunk: int) -> int:
    return min(CHUNK, cfg["tokens"] - chunk * CHUNK)


def _chunk_values(cfg: dict, tensor: int, b: int, h: int, chunk: int, std_h: np.ndarray,
                  seed: int) -> np.ndarray:
    n = _chunk_rows(cfg, chunk)
    D = cfg["head_dim"]
    z = _rng(seed, tensor, b, h, chunk).standard_normal((n, D))
    scale = std_h if tensor == TENSOR_K else np.ones(D)
    x = z * scale
    if cfg.get("inject", False):
        r = _rng(seed, TENSOR_INJECT, b, h, chunk, tensor)
        mask = r.random((n, D)) < 0.01
        cnt = int(mask.sum())
        t = np.clip(10.0 * r.standard_t(3, size=cnt), -200.0, 200.0)
        rows, cols = np.nonzero(mask)
        x[rows, cols] = t * scale[cols]
    return x


def gen_head(cfg: dict, tensor: int, b: int, h: int, t0: int = 0, t1: int | None = None,
             seed: int = 0, std: np.ndarray | None = None) -> np.ndarray:
    """fp16 bit patterns ``uint16 [t1-t0][D]`` of K (tensor 0) or V (tensor 1) for one (b, h)."""
    if t1 is None:
        t1 = cfg["tokens"]
    assert 0 <= t0 <= t1 <= cfg["tokens"]
    if std is None:
        std = chan_std(cfg, seed)
    D = cfg["head_dim"]
    out = np.empty((t1 - t0, D), np.uint16)
    c0, c1 = t0 // CHUNK, (max(t1, 1) - 1) // CHUNK
    for c in range(c0, c1 + 1):
        if t1 <= t0:
            break
        lo, hi = max(t0, c * CHUNK), min(t1, (c + 1) * CHUNK)
        if lo >= hi:
            continue
        vals = _chunk_values(cfg, tensor, b, h, c, std[h], seed)
        out[lo - t0:hi - t0] = vals[lo - c * CHUNK:hi - c * CHUNK].astype(np.float16).view(np.uint16)
    return out


def _gen_task(args):
    cfg, tensor, b, h, t0, t1, seed, std = args
    return b, h, gen_head(cfg, tensor, b, h, t0, t1, seed, std)


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gen_tensor(cfg: dict, tensor: int, t0: int = 0, t1: int | None = None, seed: int = 0,
               workers: int | None = None, out: np.ndarray | None = None,
               heads: list | None = None) -> np.ndarray:
    """fp16 bits ``uint16 [B][Hkv][t1-t0][D]`` of K or V for every (b, h), or
    ``uint16 [n][t1-t0][D]`` for the n (b, h) pairs listed in ``heads``.

    Large tensors are drawn by a pool of worker processes, one (b, h) per task;
    the result does not depend on the number of workers.
    """
    if t1 is None:
        t1 = cfg["tokens"]
    B, H, D = cfg["batch"], cfg["kv_heads"], cfg["head_dim"]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    if out is None:
        out = np.empty((B, H, t1 - t0, D) if heads is None else (len(pairs), t1 - t0, D), np.uint16)
    slot = {bh: i for i, bh in enumerate(pairs)}
    put = (lambda b, h, arr: out.__setitem__((b, h), arr)) if heads is None else \
        (lambda b, h, arr: out.__setitem__(slot[(b, h)], arr))
    std = chan_std(cfg, seed)
    tasks = [(cfg, tensor, b, h, t0, t1, seed, std) for (b, h) in pairs]
    nw = default_workers() if workers is None else workers
    if nw <= 1 or len(pairs) * (t1 - t0) * D < (1 << 22):
        for task in tasks:
            b, h, arr = _gen_task(task)
            put(b, h, arr)
        return out
    ctx = _mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=nw, mp_context=ctx) as ex:
        for b, h, arr in ex.map(_gen_task, tasks, chunksize=1):
            put(b, h, arr)
    return out


def gen_q(cfg: dict, seed: int = 0) -> np.ndarray:
    """Decode queries, fp16 bits ``uint16 [B][Hq][D]`` (pre-RoPE)."""
    B, Hq, D = cfg["batch"], cfg["q_heads"], cfg["head_dim"]
    out = np.empty((B, Hq, D), np.uint16)
    for b in range(B):
        out[b] = _rng(seed, TENSOR_Q, b).standard_normal((Hq, D)).astype(np.float16).view(np.uint16)
    return out


def gen_q_chunk(cfg: dict, nq: int, seed: int = 0) -> np.ndarray:
    """Queries of a chunk of ``nq`` tokens, fp16 bits ``uint16 [B][Hq][nq][D]``
    (pre-RoPE), drawn like the decode queries from N(0, 1)."""
    B, Hq, D = cfg["batch"], cfg["q_heads"], cfg["head_dim"]
    out = np.empty((B, Hq, nq, D), np.uint16)
    for b in range(B):
        out[b] = _rng(seed, TENSOR_QCHUNK, b, nq).standard_normal((Hq, nq, D)).astype(np.float16).view(np.uint16)
    return out


def _lloyd_1d(x: np.ndarray, k: int, iters: int = 100) -> np.ndarray:
    """1-D Lloyd k-means in float64 on one sample ``x``: initial centres at the
    (j + 0.5)/k sample quantiles; each point joins the nearest centre, split at the
    midpoints between sorted centres with a point on a midpoint joining the lower
    centre; an empty cluster keeps its centre; at most ``iters`` rounds, stopping
    once no assignment changes."""
    xs = np.sort(x)
    cs = np.concatenate([[0.0], np.cumsum(xs)])
    c = np.quantile(xs, (np.arange(k) + 0.5) / k)
    bounds = None
    for _ in range(iters):
        mids = (c[:-1] + c[1:]) * 0.5
        b = np.concatenate([[0], np.searchsorted(xs, mids, side="right"), [xs.size]])
        if bounds is not None and np.array_equal(b, bounds):
            break
        bounds = b
        cnt = b[1:] - b[:-1]
        nz = cnt > 0
        c[nz] = (cs[b[1:]] - cs[b[:-1]])[nz] / cnt[nz]
        c = np.sort(c)
    return c


def calib_lut(cfg: dict, seed: int = 1, ntok: int = 4096) -> np.ndarray:
    """Per-(kv-head, channel) non-uniform codebook, fp16 bits ``uint16 [Hkv][D][2**k_bits]``,
    sorted ascending along the last axis."""
    H, D, K = cfg["kv_heads"], cfg["head_dim"], 1 << cfg["k_bits"]
    std = chan_std(cfg, 0)
    out = np.empty((H, D, K), np.uint16)
    for h in range(H):
        x = _rng(seed, TENSOR_CALIB, h).standard_normal((ntok, D)) * std[h]
        for d in range(D):
            c16 = np.sort(_lloyd_1d(x[:, d], K).astype(np.float16))
            out[h, d] = c16.view(np.uint16)
    return out


def _value_calib_sample(cfg: dict, h: int, seed: int, ntok: int) -> np.ndarray:
    """A seeded calibration sample of one kv head's values, float64 ``[ntok][D]``, drawn
    like the workload's values (N(0, 1) per element)."""
    return _rng(seed, TENSOR_VCALIB, h).standard_normal((ntok, cfg["head_dim"]))


def calib_vlut(cfg: dict, seed: int = 2, ntok: int = 4096) -> np.ndarray:
    """Per-(kv-head, channel) non-uniform value codebook, fp16 bits
    ``uint16 [Hkv][D][2**v_bits]``, sorted ascending: 1-D Lloyd k-means per channel on a
    calibration sample, as the offline calibration of the key codebook."""
    H, D, K = cfg["kv_heads"], cfg["head_dim"], 1 << cfg["v_bits"]
    out = np.empty((H, D, K), np.uint16)
    for h in range(H):
        x = _value_calib_sample(cfg, h, seed, ntok)
        for d in range(D):
            out[h, d] = np.sort(_lloyd_1d(x[:, d], K).astype(np.float16)).view(np.uint16)
    return out


def log_vlut(cfg: dict, absmax: np.ndarray) -> np.ndarray:
    """Log-spaced value codebook, fp16 bits ``uint16 [Hkv][D][2**v_bits]``, sorted
    ascending: the levels +-s 2^-k for k < 2^(v_bits - 1), with s = absmax[h][d] rounded
    to fp16 (so every level is an fp16 number unless it falls below the normal range)."""
    H, D, K = cfg["kv_heads"], cfg["head_dim"], 1 << cfg["v_bits"]
    half = K // 2
    s = np.asarray(absmax, np.float64).reshape(H, D).astype(np.float16).astype(np.float64)
    pos = s[:, :, None] * 2.0 ** -np.arange(half)[::-1]                 # ascending
    lv = np.concatenate([-pos[:, :, ::-1], pos], axis=2)
    return lv.astype(np.float16).view(np.uint16)


def calib_log_vlut(cfg: dict, seed: int = 2, ntok: int = 4096, q: float = 0.999) -> np.ndarray:
    """log_vlut with s the q-quantile of |x| per channel of the calibration sample."""
    H = cfg["kv_heads"]
    absmax = np.stack([np.quantile(np.abs(_value_calib_sample(cfg, h, seed, ntok)), q, axis=0) for h in range(H)])
    return log_vlut(cfg, absmax)
