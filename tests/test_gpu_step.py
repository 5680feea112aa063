"""GPU parity of the fused decode step (kvq_decode_step: append one token per sequence and
attend at its position; the token is read from the input and stored into the tail by the
attention's own kernels, and a completed block is quantized first).

From a cache of T0 tokens, N steps run token by token across a block boundary.  Every
step's output must be within 2e-3 of the oracle's fp64 decode over a cache built from the
first t + 1 tokens (the step's own token included), and after the last step the cache
buffers must equal the oracle's bit for bit.  The same steps through kvq_quantize_append
and kvq_decode_attention give the same outputs up to fp32 rounding.

Split count 0 is the library's choice: the one-launch kernel for a short cache (at most
four quantized blocks) in a configuration no tuned kernel covers (mha_k3, and gqa_d64
until its fifth block, where it changes over), else the split kernels (tuned MHA or GQA,
or the generic one for gqa_d64_long and the kept-key cases) and the finish kernel.  Split count 3 forces the
split kernels.
"""
import numpy as np
import pytest

import synth
from _gpu_util import build_gpu_cache, compare_head, inputs, say, upload

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import quantized_decode_attn_amd as kvq
    kvq.lib()
    import oracle
    oracle.build()


CASES = {
    "c0_tiny": (synth.config("c0", tokens=200, capacity=256), 110),
    "mha_d128": (synth.config("c1", batch=2, q_heads=2, kv_heads=2, tokens=3 * 128 + 20, capacity=512), 120),
    "gqa_csr": (synth.config("c2", batch=1, q_heads=8, kv_heads=2, tokens=2 * 128 + 100, capacity=512), 40),
    "lut3_v2": (synth.config("c3", batch=1, q_heads=2, kv_heads=2, tokens=2 * 128 + 120, capacity=512), 12),
    "clip_csr": (synth.config("c4", batch=1, q_heads=2, kv_heads=2, tokens=128 + 125, capacity=384), 6),
    # past eight blocks per sequence: two launches even at split count 0
    "mha_long": (synth.config("c1", batch=1, q_heads=2, kv_heads=2, tokens=10 * 128 + 60, capacity=1408), 80),
    "gqa_long": (synth.config("c2", batch=1, q_heads=8, kv_heads=2, tokens=9 * 128 + 20, capacity=1280), 30),
    "d64_long": (synth.config("c0", tokens=9 * 64 + 10, capacity=640), 20),
    # no tuned kernel: head_dim 64 with grouped queries, 3-bit uniform keys
    "gqa_d64": (synth.config("c0", q_heads=8, kv_heads=2, tokens=5 * 64 + 30, capacity=384), 40),
    "mha_k3": (synth.config("c1", batch=1, q_heads=2, kv_heads=2, k_bits=3, tokens=3 * 128 + 20, capacity=512), 30),
    "gqa_d64_long": (synth.config("c0", q_heads=8, kv_heads=2, tokens=9 * 64 + 10, capacity=640), 20),
    # keys kept in fp16 by norm: the quantize of a completed block picks them
    "mha_keep": (synth.config("c1", batch=1, q_heads=2, kv_heads=2, tokens=3 * 128 + 20, capacity=512,
                              keep_pct=5), 40),
    "gqa_d64_keep": (synth.config("c0", q_heads=8, kv_heads=2, tokens=5 * 64 + 30, capacity=384,
                                  keep_pct=12), 40),
}


def _lut(cfg):
    return synth.calib_lut(cfg) if cfg["k_mode"] == 1 else None


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("case", sorted(CASES))
def test_fused_steps_match_oracle_and_two_calls(case, splits):
    import torch
    import oracle
    cfg, n_steps = CASES[case]
    T = cfg["tokens"]
    T0 = T - n_steps
    B, H, Hq = cfg["batch"], cfg["kv_heads"], cfg["q_heads"]
    gq = Hq // H
    say("case", case, "splits", splits, "T0", T0, "steps", n_steps)
    k, v = inputs(cfg)
    lut = _lut(cfg)
    qs = synth.gen_q_chunk(cfg, n_steps)                      # step i's query: qs[:, :, i]
    fused = build_gpu_cache(cfg, k[:, :, :T0], v[:, :, :T0], None, lut)
    plain = build_gpu_cache(cfg, k[:, :, :T0], v[:, :, :T0], None, lut)
    kd, vd, qd = upload(k), upload(v), upload(qs)
    worst, worst_pair = 0.0, 0.0
    for i in range(n_steps):
        t = T0 + i
        k1, v1, q1 = kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), qd[:, :, i].contiguous()
        a = fused.step(k1, v1, q1, num_splits=splits).cpu().numpy().astype(np.float64)
        plain.append(kd[:, :, t:t + 1].contiguous(), vd[:, :, t:t + 1].contiguous())
        d = plain.decode(q1, q_pos=t).cpu().numpy().astype(np.float64)
        assert fused.length == t + 1 == plain.length
        # oracle: a cache of the first t + 1 tokens, decoded at position t
        cfg_t = dict(cfg, tokens=t + 1)
        hl, ql = [], []
        heads = {}
        for b in range(B):
            for h in range(H):
                heads[(b, h)] = oracle.HeadCache(cfg_t, None if lut is None else lut[h]).build(
                    k[b, h, :t + 1], v[b, h, :t + 1])
        for b in range(B):
            for hq in range(Hq):
                hl.append(heads[(b, hq // gq)])
                ql.append(qs[b, hq, i])
        ref = oracle.decode_many(cfg_t, hl, np.stack(ql), t).reshape(B, Hq, -1)
        worst = max(worst, float(np.abs(a - ref).max()))
        worst_pair = max(worst_pair, float(np.abs(a - d).max()))
    say("  max abs err vs oracle", worst, "vs append + decode", worst_pair)
    assert worst <= TOL
    assert worst_pair <= 1e-4
    torch.cuda.synchronize()
    ko = oracle.kout(cfg)
    for b in range(B):
        for h in range(H):
            hc = oracle.HeadCache(cfg, None if lut is None else lut[h]).build(k[b, h], v[b, h])
            compare_head(fused, hc, cfg, ko, b, h)


def test_step_rejects_a_full_cache():
    import quantized_decode_attn_amd as kvq
    cfg = synth.config("c0", tokens=128, capacity=128)
    k, v = inputs(cfg)
    cache = build_gpu_cache(cfg, k, v)
    k1, v1 = upload(k[:, :, 0]), upload(v[:, :, 0])
    q = upload(synth.gen_q(cfg))
    with pytest.raises(kvq.KvqError):
        cache.step(k1, v1, q)
    assert cache.length == 128


@pytest.mark.parametrize("case,splits", [("gqa_d64", 0), ("c0_tiny", 3)])
def test_steps_replay_as_a_graph(case, splits):
    """A run of steps captured as one HIP graph (a serving loop's use) and replayed three
    times, the cache buffers restored to the run's starting state before each replay
    (the steps overwrite tail slots the first steps read): every replay gives the eager
    run's outputs bit for bit and leaves the same cache."""
    import torch
    cfg = CASES[case][0]
    n = 80                                             # crosses a block boundary
    T = cfg["tokens"]
    T0 = T - n
    B, H, Hq, D = cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["head_dim"]
    k, v = inputs(cfg)
    qs = synth.gen_q_chunk(cfg, n)
    kd, vd, qd = upload(k), upload(v), upload(qs)
    toks = [(kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), qd[:, :, t - T0].contiguous())
            for t in range(T0, T)]
    eager = build_gpu_cache(cfg, k[:, :, :T0], v[:, :, :T0], None, _lut(cfg))
    ref = torch.stack([eager.step(a, b, c, num_splits=splits) for a, b, c in toks])
    torch.cuda.synchronize()
    cache = build_gpu_cache(cfg, k[:, :, :T0], v[:, :, :T0], None, _lut(cfg))
    cache.workspace(splits)
    outs = torch.empty((n, B, Hq, D), dtype=torch.float32, device=kd.device)
    start = {name: buf.clone() for name, buf in cache.bufs.items() if buf is not None}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
            for i, (a, b, c) in enumerate(toks):
                cache.step(a, b, c, num_splits=splits, out=outs[i], stream=side)
    assert cache.length == T
    for r in range(3):
        outs.fill_(float("nan"))
        for name, buf in start.items():
            cache.bufs[name].copy_(buf)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("replay", r, "max abs diff", float((outs - ref).abs().max()))
        assert torch.equal(outs, ref), r
        eager.decode(toks[-1][2])                      # eager work between replays
        torch.cuda.synchronize()
    import oracle
    lut = _lut(cfg)
    ko = oracle.kout(cfg)
    for b in range(B):
        for h in range(H):
            hc = oracle.HeadCache(cfg, lut).build(k[b, h], v[b, h])
            compare_head(cache, hc, cfg, ko, b, h)
