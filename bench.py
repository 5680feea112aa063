"""Benchmark of the low-bit KV-cache hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: the
quantize-append of the batch's new keys and values into the cache (every block
quantized, clipped, split into dense codes and outlier CSR, packed, with its
metadata) followed by one decode-attention query per sequence over the packed cache.
The default workload is the prefill-append one: 16 sequences x 32 kv heads, 16384 new
tokens appended onto 16384 cached ones, 99th-percentile clip, 1% outliers, then a
decode over all 32768 tokens.  Inputs are resident in HBM before timing starts.
``value`` is the decode attention's effective bandwidth (algorithmic bytes over the
decode call's average duration, measured with HIP events on the stream the kernels
run on); the append's tokens/s is reported beside it, as is a read-streaming probe
(the achievable bandwidth of a plain 1 GiB read on the same device and stream).

    python bench.py [--steps K] [--warmup W] [--workload c4] [--gpus 1] [--chunk NQ]

``--chunk NQ`` adds a third timed call to every step: causal attention of a chunk of NQ
queries per sequence at the newest NQ positions (a prefill chunk or speculative
verification) over the same cache, reported under "chunk".

``--decode-steps N`` also times token-by-token generation on a second cache holding the
workload's first T - N tokens: N fused decode steps (kvq_decode_step: the token appended
inside the attention's own launches), then the same N tokens as kvq_quantize_append of one token
followed by kvq_decode_attention; reported per step under "decode_step".

``--paged`` also times the workload's shapes as a continuous batch: per-sequence lengths
in [T/8, T], blocks in a shuffled pool of exactly the blocks they need; the ragged
prefill (kvq_quantize_append_seqs) and the decode of every sequence at its own newest
token, paged and in dense slots; reported under "paged".

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E, published
METRIC = "int4-KV decode attention GB/s & frac of HBM peak; quantize-append tokens/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kout(cfg):
    p = cfg["outlier_pct"]
    return (p * cfg["head_dim"] + 99) // 100 if p > 0 else 0


def keep_count(cfg) -> int:
    p = cfg.get("keep_pct", 0)
    return (p * cfg["k_block"] + 99) // 100 if p > 0 else 0


def decode_bytes_per_token_head(cfg) -> float:
    """Bytes one decode must read per (b, kv-head, token): packed key and value codes,
    key scale/zero amortised over the block, value scale/zero, outlier columns and
    values, and the keys kept in fp16 (one offset byte and 2 D bytes each, amortised
    over the block).  The CSR row pointers (4 B per token and tensor) are not counted:
    every quantized token holds exactly ceil(pct * D / 100) entries, so a reader
    computes the offsets and never loads the pointers."""
    D, Bk, ko = cfg["head_dim"], cfg["k_block"], kout(cfg)
    rk = D * cfg["k_bits"] / 8
    rv = D * cfg["v_bits"] / 8
    kmeta = 2 * D * 2 / Bk if cfg["k_mode"] == 0 else 0.0
    vmeta = (D // cfg["v_group"]) * 2 * 2 if cfg.get("v_mode", 0) == 0 else 0.0
    csr = 2 * ko * 3
    kept = keep_count(cfg) * (1 + 2 * D) / Bk
    return rk + rv + kmeta + vmeta + csr + kept


def decode_bytes(cfg, T) -> float:
    B, H, Hq, D = cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["head_dim"]
    lut = H * D * (1 << cfg["k_bits"]) * 2 if cfg["k_mode"] == 1 else 0
    lut += H * D * (1 << cfg["v_bits"]) * 2 if cfg.get("v_mode", 0) == 1 else 0
    return B * H * T * decode_bytes_per_token_head(cfg) + B * Hq * D * (2 + 4) + lut


def append_bytes_per_token_head(cfg) -> float:
    """fp16 keys and values read, packed codes, scale/zero and outlier CSR written."""
    D, ko = cfg["head_dim"], kout(cfg)
    csr = 2 * (ko * 3 + 4) if ko else 0
    return 2 * D * 2 + decode_bytes_per_token_head(cfg) - 2 * ko * 3 + csr


def dtype_of(cfg) -> str:
    """The arithmetic the decode computes in, for the JSON line."""
    if cfg.get("v_mode", 0) == 2:
        return "f32 scores/softmax over E4M3 keys and values (exact conversions); fp32 accumulation"
    if cfg.get("v_mode", 0) == 1:
        return "f32 scores/softmax; fp16 codebook values times f32 probabilities; fp32 accumulation"
    w = "30-bit digit" if cfg["q_heads"] > cfg["kv_heads"] else "24-bit"
    return ("f32 scores/softmax; value weights as %s fixed point x u%d codes, exact integer sums; "
            "fp32 accumulation" % (w, cfg["v_bits"]))


def source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantized_decode_attn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str, workload: str, src_hash: str, nq: int | None = None):
    """HBM bytes per call from the committed counter summary, if it was taken on this
    workload (and chunk size) and on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        recs = json.load(open(path))["records"]
    except (OSError, KeyError, ValueError):
        return None
    for rec in recs:
        if (rec.get("kind") == kind and rec.get("workload") == workload
                and rec.get("source_hash") == src_hash and rec.get("nq") == nq):
            return rec.get("bytes_per_launch")
    return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, k, v, q, lut, seconds: float, vlut=None):
    """The oracle as it stands, on a bounded sample of the same workload: quantize a
    sample of heads (OpenMP across heads), then time fp64 decode over them; each leg
    is sized to about ``seconds`` of wall time."""
    import oracle
    oracle.build()
    T, D, Hq, H = cfg["tokens"], cfg["head_dim"], cfg["q_heads"], cfg["kv_heads"]
    B = cfg["batch"]
    gq = Hq // H
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    hc = oracle.HeadCache(cfg, None if lut is None else lut[0], None if vlut is None else vlut[0]).build(k[0, 0], v[0, 0])
    t_build1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.decode_many(cfg, [hc], q[0, :1], T - 1)
    t_dec1 = time.perf_counter() - t0
    per = max(t_build1, gq * t_dec1, 1e-3)
    nheads = int(max(1, min(B * H, seconds * threads / per)))
    sample = [(i // H, i % H) for i in range(nheads)]
    ks = np.stack([k[b, h] for (b, h) in sample])
    vs = np.stack([v[b, h] for (b, h) in sample])
    luts = None if lut is None else [lut[h] for (_, h) in sample]
    vluts = None if vlut is None else [vlut[h] for (_, h) in sample]
    t0 = time.perf_counter()
    heads = oracle.build_heads(cfg, ks, vs, luts, vluts)
    t_build = time.perf_counter() - t0
    del ks, vs
    hl = [heads[i] for i in range(nheads) for _ in range(gq)]
    ql = np.stack([q[b, h * gq + g] for (b, h) in sample for g in range(gq)])
    t0 = time.perf_counter()
    oracle.decode_many(cfg, hl, ql, T - 1)
    t_dec = time.perf_counter() - t0
    dec_bytes = nheads * T * decode_bytes_per_token_head(cfg)
    return {
        "value": round(dec_bytes / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "%d of %d (b, kv-head) heads x %d tokens: quantized by the oracle in %.1f s "
                  "(%.3g tokens/s), then fp64 decode of %d query heads each in %.1f s"
                  % (nheads, B * H, T, t_build, nheads * T / t_build, gq, t_dec),
        "append_tokens_per_s": round(nheads * T / t_build, 1),
    }


def copy_probe():
    """A plain 1 GiB device-to-device copy (for scaling HBM byte counters)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("copy probe: 3 x %d bytes" % n)


def time_decode_steps(cfg, k_d, v_d, lut_d, n, dev):
    """Per-step time of n token-by-token decode steps on a cache of the workload's first
    T - n tokens, three ways: kvq_decode_step with the library's choice of kernels (one
    launch for a short cache), kvq_decode_step on the split kernels, and
    kvq_quantize_append of one token followed by kvq_decode_attention.  Each is timed with
    HIP events over the whole run, once issued call by call from Python (host cost
    included) and once captured as one HIP graph of the n steps and replayed (the cost on
    the GPU: kernels and the gaps between launches), the cache buffers restored to the
    starting state before each replay, outside the timed region."""
    import torch
    import quantized_decode_attn_amd as kvq
    T, B, Hq, D = cfg["tokens"], cfg["batch"], cfg["q_heads"], cfg["head_dim"]
    T0 = T - n
    qs = torch.from_numpy(np.ascontiguousarray(synth.gen_q_chunk(cfg, n)).view(np.int16)).to(dev).view(torch.float16)
    toks_k = [k_d[:, :, t].contiguous() for t in range(T0, T)]
    toks_v = [v_d[:, :, t].contiguous() for t in range(T0, T)]
    toks_k1 = [k_d[:, :, t:t + 1].contiguous() for t in range(T0, T)]
    toks_v1 = [v_d[:, :, t:t + 1].contiguous() for t in range(T0, T)]
    q1 = [qs[:, :, i].contiguous() for i in range(n)]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    cache = kvq.Cache(cfg, device=dev, lut=lut_d)
    # the library's split count, read back from its workspace size
    s_auto = kvq.kvq_decode_workspace_bytes(cache.desc, 0) // (B * Hq * (D + 2) * 4)
    cache.workspace(s_auto)

    def reset():
        cache.desc.length = 0
        cache.append(k_d[:, :, :T0].contiguous(), v_d[:, :, :T0].contiguous())
        torch.cuda.synchronize()

    def run(mode, stream):
        for i in range(n):
            if mode == "fused":
                cache.step(toks_k[i], toks_v[i], q1[i], out=out, stream=stream)
            elif mode == "fused_split":
                cache.step(toks_k[i], toks_v[i], q1[i], num_splits=s_auto, out=out, stream=stream)
            else:
                cache.append(toks_k1[i], toks_v1[i], stream=stream)
                cache.decode(q1[i], q_pos=T0 + i, out=out, stream=stream)

    modes = ("fused", "fused_split", "two_calls")
    eager, graph = {}, {}
    stream = torch.cuda.current_stream()
    for mode in modes + modes:   # each twice; the second run is reported
        reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(mode, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        eager[mode] = e0.elapsed_time(e1) * 1e3 / n
    replays = 5
    for mode in modes:
        reset()
        start = {name: buf.clone() for name, buf in cache.bufs.items() if buf is not None}
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
                run(mode, side)
        torch.cuda.synchronize()
        total = 0.0
        for r in range(replays + 1):        # the first replay warms up
            for name, buf in start.items():
                cache.bufs[name].copy_(buf)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            if r:
                total += e0.elapsed_time(e1)
        graph[mode] = total * 1e3 / (n * replays)
        del g
    log("decode step, us/token issued from Python: fused %.1f (split kernels %.1f), append + decode %.1f"
        % (eager["fused"], eager["fused_split"], eager["two_calls"]))
    log("decode step, us/token replayed as a graph: fused %.1f (split kernels %.1f), append + decode %.1f "
        "(%d tokens from %d)" % (graph["fused"], graph["fused_split"], graph["two_calls"], n, T0))
    r2 = lambda x: round(x, 2)
    return {"tokens": n, "from_length": T0, "splits": int(s_auto),
            "graph_us_per_token": {k: r2(v) for k, v in graph.items()},
            "python_us_per_token": {k: r2(v) for k, v in eager.items()},
            "graph_speedup_vs_append_plus_decode": round(graph["two_calls"] / graph["fused"], 3)}


def time_paged(cfg, k_d, v_d, lut_d, dev, reps=10):
    """The workload's shapes as a continuous batch: per-sequence lengths drawn uniformly
    from [T/8, T] (seeded), the quantized blocks in a pool of exactly the blocks they
    need, mapped through a shuffled block table.  Times the ragged prefill (one
    kvq_quantize_append_seqs of every sequence's tokens) and the decode of every sequence
    at its own newest token, against the same lengths in the dense slots."""
    import torch
    import quantized_decode_attn_amd as kvq
    T, B, H, Hq, D, Bk = (cfg["tokens"], cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["head_dim"],
                          cfg["k_block"])
    rng = np.random.default_rng(11)
    lengths = rng.integers(T // 8, T + 1, size=B)
    need = [-(-int(L) // Bk) for L in lengths]
    P = int(sum(need))
    perm = rng.permutation(P)
    table = np.zeros((B, T // Bk), np.int32)
    i = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[i:i + n]
        i += n
    q = torch.from_numpy(np.ascontiguousarray(synth.gen_q(cfg, seed=4)).view(np.int16)).to(dev).view(torch.float16)
    kin, vin = k_d[:, :, :T].contiguous(), v_d[:, :, :T].contiguous()
    tokens = int(lengths.sum())
    dbytes = tokens * H * decode_bytes_per_token_head(cfg) + B * Hq * D * 6
    abytes = tokens * H * append_bytes_per_token_head(cfg)
    res = {"lengths": "uniform in [T/8, T], seed 11", "tokens": tokens, "pool_blocks": P,
           "pool_fraction_of_dense": round(P / (B * T / Bk), 3)}
    stream = torch.cuda.current_stream()
    for name, paged in (("paged", True), ("dense_slots", False)):
        if paged:
            cache = kvq.PagedCache(cfg, num_blocks=P, block_table=torch.from_numpy(table).to(dev), device=dev,
                                   lut=lut_d)
        else:
            cache = kvq.PagedCache(cfg, device=dev, lut=lut_d)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cache.append_seqs(kin, vin, lengths)
        e1.record(stream)
        torch.cuda.synchronize()
        app_us = e0.elapsed_time(e1) * 1e3
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        cache.workspace(0)
        for _ in range(2):
            cache.decode(q, out=out)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            cache.decode(q, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_us = e0.elapsed_time(e1) * 1e3 / reps
        res[name] = {"decode_us": round(dec_us, 2), "decode_GBps": round(dbytes / dec_us / 1e3, 1),
                     "decode_frac": round(dbytes / dec_us / 1e3 / HBM_PEAK_GBPS, 4),
                     "prefill_append_us": round(app_us, 1),
                     "prefill_append_tokens_per_s": round(tokens / app_us * 1e6, 1),
                     "prefill_append_GBps": round(abytes / app_us / 1e3, 1)}
        log("%-11s decode %.1f us %.0f GB/s (%.1f%% of 8 TB/s); ragged prefill append %.1f us %.0f GB/s"
            % (name, dec_us, dbytes / dec_us / 1e3, 100 * dbytes / dec_us / 1e3 / HBM_PEAK_GBPS, app_us,
               abytes / app_us / 1e3))
        del cache
    res["algorithmic_decode_bytes"] = int(dbytes)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4", choices=sorted(synth.CONFIGS))
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--chunk", type=int, default=0, help="also time attention of a chunk of this many queries")
    ap.add_argument("--chunk-splits", type=int, default=0)
    ap.add_argument("--decode-steps", type=int, default=0, help="also time this many token-by-token steps")
    ap.add_argument("--paged", action="store_true", help="also time a paged cache with mixed sequence lengths")
    ap.add_argument("--keep-pct", type=int, default=0,
                    help="the workload with this percentage of each block's keys kept in fp16 by norm")
    ap.add_argument("--fp8", action="store_true", help="the workload as an FP8 (E4M3) cache")
    ap.add_argument("--v-codebook", choices=["none", "kmeans", "log"], default="none",
                    help="the workload with values quantized by a per-channel codebook (calibrated or log-spaced)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    cfg = synth.config(args.workload)
    if args.keep_pct:
        cfg["keep_pct"] = args.keep_pct
        cfg["workload"] += "-keep%dpct" % args.keep_pct
    if args.v_codebook != "none":
        cfg["v_mode"] = 1
        cfg["workload"] += "-v%s" % args.v_codebook
    if args.fp8:
        cfg.update(k_mode=2, k_bits=8, v_mode=2, v_bits=8, outlier_pct=0, clip_quantile=0.0, inject=False)
        cfg["workload"] += "-fp8"
    T, B, H, Hq, D = cfg["tokens"], cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["head_dim"]
    existing = cfg["existing"]
    log("workload", args.workload, cfg["workload"])
    t0 = time.time()
    k = synth.gen_tensor(cfg, synth.TENSOR_K)
    v = synth.gen_tensor(cfg, synth.TENSOR_V)
    q = synth.gen_q(cfg)
    lut = synth.calib_lut(cfg) if cfg["k_mode"] == 1 else None
    vlut = None  # (an FP8 cache has no codebook)
    if args.v_codebook != "none":
        vlut = synth.calib_log_vlut(cfg) if args.v_codebook == "log" else synth.calib_vlut(cfg)
    log("inputs drawn in %.1f s" % (time.time() - t0))

    import torch
    import quantized_decode_attn_amd as kvq
    kvq.lib()
    dev = torch.device("cuda:0")
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.float16)
    k_d, v_d, q_d = up(k), up(v), up(q)
    lut_d = None if lut is None else torch.from_numpy(lut.view(np.int16)).to(dev)
    vlut_d = None if vlut is None else torch.from_numpy(vlut.view(np.int16)).to(dev)
    cache = kvq.Cache(cfg, device=dev, lut=lut_d, vlut=vlut_d)
    if existing:
        cache.append(k_d[:, :, :existing].contiguous(), v_d[:, :, :existing].contiguous())
    k_new = k_d[:, :, existing:].contiguous()
    v_new = v_d[:, :, existing:].contiguous()
    n_new = T - existing
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    cache.workspace(args.splits)
    nq = args.chunk
    if nq:
        qc_d = up(synth.gen_q_chunk(cfg, nq))
        outc = torch.empty((B, Hq, nq, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    # Untimed between the timed regions: a 1 GiB read that evicts the 256 MB Infinity
    # Cache and the L2 (writing back the append's dirty lines), so that neither the append
    # nor the decode starts with the other's data, or dirty lines, in the caches.
    scrub = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    scrub_view = scrub.view(torch.int64)      # summed as stored: no widened copy

    def step(e=None):
        cache.desc.length = existing            # re-append the same tokens into the same slots
        scrub_view.sum()
        if e: e[0].record(stream)
        cache.append(k_new, v_new)
        if e: e[1].record(stream)
        scrub_view.sum()
        if e: e[2].record(stream)
        cache.decode(q_d, q_pos=T - 1, num_splits=args.splits, out=out)
        if e: e[3].record(stream)
        if nq:
            scrub_view.sum()
            if e: e[4].record(stream)
            cache.chunk(qc_d, q_pos=T - nq, num_splits=args.chunk_splits, out=outc)
            if e: e[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    app_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)])
    dec_ms = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(args.steps)])

    # read-streaming probe: the same 1 GiB int64 sum that scrubs the caches, timed on
    # the same stream (achievable read bandwidth of this device, for the fraction below)
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for r in range(5):
        pe[r].record(stream)
        scrub_view.sum()
    pe[5].record(stream)
    torch.cuda.synchronize()
    probe_ms = np.array([pe[r].elapsed_time(pe[r + 1]) for r in range(1, 5)])
    probe_gbps = scrub.numel() / (probe_ms.mean() * 1e-3) / 1e9

    dbytes = decode_bytes(cfg, T)
    abytes = B * H * n_new * append_bytes_per_token_head(cfg)
    dec_gbps = dbytes / (dec_ms.mean() * 1e-3) / 1e9
    app_gbps = abytes / (app_ms.mean() * 1e-3) / 1e9
    app_tps = B * n_new / (app_ms.mean() * 1e-3)
    log("decode  %.1f us  %.1f GB/s (%.1f%% of 8 TB/s)" % (dec_ms.mean() * 1e3, dec_gbps, dec_gbps / 80))
    log("append  %.1f us  %.1f GB/s  %.3g tokens/s" % (app_ms.mean() * 1e3, app_gbps, app_tps))
    log("stream  %.1f GB/s (1 GiB read probe)" % probe_gbps)

    dec_hash = source_hash(["decode_mha.hip", "decode_gqa.hip", "decode_common.h", "decode.hip",
                            "kvq_device.h", "kvq_internal.h"])
    app_hash = source_hash(["quantize.hip", "quantize_block.h", "quantize_keys.hip", "quantize_keys_lut.hip",
                            "quantize_values.hip", "kvq_device.h", "kvq_internal.h"])
    tr_dec = measured_traffic("decode", cfg["workload"], dec_hash)
    tr_app = measured_traffic("append", cfg["workload"], app_hash)
    rec = {
        "metric": METRIC,
        "value": round(dec_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_of(cfg),
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": cfg["workload"], "batch": B, "q_heads": Hq, "kv_heads": H,
                   "head_dim": D, "tokens": T, "appended_per_step": n_new, "k_bits": cfg["k_bits"],
                   "v_bits": cfg["v_bits"], "k_block": cfg["k_block"], "v_group": cfg["v_group"],
                   "splits": args.splits or "auto", "keep_pct": cfg.get("keep_pct", 0),
                   "v_mode": cfg.get("v_mode", 0)},
        "frac_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "decode_us": round(float(dec_ms.mean()) * 1e3, 2),
        "append_us": round(float(app_ms.mean()) * 1e3, 2),
        "append_tokens_per_s": round(app_tps, 1),
        "append_GBps": round(app_gbps, 2),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": tr_dec, "kernel": "decode (split + combine launches)",
                     "algorithmic_bytes": int(dbytes)},
        "roofline_append": {"bound": "hbm", "achieved": round(app_gbps, 2), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(app_gbps / HBM_PEAK_GBPS, 4),
                            "traffic": tr_app, "kernel": "append (key and value quantize launches)",
                            "algorithmic_bytes": int(abytes)},
        "stream_probe": {"GBps": round(probe_gbps, 1), "frac_of_peak": round(probe_gbps / HBM_PEAK_GBPS, 4),
                         "kernel": "1 GiB int64 sum (read-streaming)"},
        "decode_frac_of_stream": round(dec_gbps / probe_gbps, 4),
        "append_frac_of_stream": round(app_gbps / probe_gbps, 4),
    }
    if nq:
        ch_ms = np.array([ev[i][4].elapsed_time(ev[i][5]) for i in range(args.steps)])
        cbytes = B * H * T * decode_bytes_per_token_head(cfg) + B * Hq * nq * D * (2 + 4)
        # QK and PV: 2 D flops each per (query, visible token)
        vis = sum(min(T - nq + j + 1, T) for j in range(nq))
        cflops = 4.0 * B * Hq * D * vis
        c_gbps = cbytes / (ch_ms.mean() * 1e-3) / 1e9
        c_tflops = cflops / (ch_ms.mean() * 1e-3) / 1e12
        log("chunk   %.1f us  nq %d  %.1f GB/s (%.1f%% of 8 TB/s)  %.1f TFLOP/s"
            % (ch_ms.mean() * 1e3, nq, c_gbps, c_gbps / 80, c_tflops))
        ch_hash = source_hash(["chunk_mfma.hip", "decode.hip", "decode_common.h", "kvq_device.h", "kvq_internal.h"])
        rec["chunk"] = {"nq": nq, "q_pos": T - nq, "splits": args.chunk_splits or "auto",
                        "us": round(float(ch_ms.mean()) * 1e3, 2),
                        "GBps": round(c_gbps, 2), "frac_hbm_peak": round(c_gbps / HBM_PEAK_GBPS, 4),
                        "TFLOPs": round(c_tflops, 2), "algorithmic_bytes": int(cbytes),
                        "algorithmic_flops": cflops,
                        "query_tokens_per_s": round(B * nq / (ch_ms.mean() * 1e-3), 1),
                        "kernel": "chunk (split + finish launches)",
                        "traffic": measured_traffic("chunk", cfg["workload"], ch_hash, nq)}
    if args.decode_steps:
        rec["decode_step"] = time_decode_steps(cfg, k_d, v_d, lut_d, args.decode_steps, dev)
    if args.paged:
        rec["paged"] = time_paged(cfg, k_d, v_d, lut_d, dev)
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(cfg, k, v, q, lut, args.cpu_seconds, vlut)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
