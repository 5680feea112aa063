"""GPU parity on the quantizer's degenerate cases and on very many decode splits.

* Exact ties: value rows and key channels whose group minimum and maximum make the
  scale a power of two, with members at (k + 1/2) steps, so the quotient (x - z) / s is
  an exact half-integer and the code is decided by round-half-to-even (the exact
  branch of the kernels' code step).  With and without the percentile clip and the
  outlier split.
* Constant groups (scale 0: every code 0, x = zero-point) and empty key channels
  (every member of a channel is an outlier), with and without the clip.
* Decode with 1024 and 4096 splits per kv head on a cache of 1024 blocks: the long
  context workload's "at least 1024 chunks", including 3072 splits with no block.

Caches are compared with the oracle bit for bit; decode outputs within 2e-3, and
decodes that differ only in their split count within the fp32 rounding bound
``split_tol`` (derived in the design notes: both results are fp32 evaluations of the
same sum, with at most nblk + S + 32 roundings of u = 2^-24 on terms bounded by
max |v|, counted twice).
"""
import numpy as np
import pytest

import synth
from _gpu_util import build_gpu_cache, compare_head, oracle_heads, say, upload

pytestmark = pytest.mark.gpu

TOL = 2e-3
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import quantized_decode_attn_amd as kvq
    kvq.lib()
    import oracle
    oracle.build()


def split_tol(vmax, nblk, s1, s2):
    return 4.0 * U * vmax * (nblk + s1 + s2 + 32)


def f16(x):
    return np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float16)).view(np.uint16)


def tie_inputs(cfg, seed=5):
    """Values: every row holds its group minimum z, maximum z + 15 s (s a power of two)
    and members z + (k + 1/2) s; keys: every block and channel holds the same pattern
    along its tokens.  Both at random signs and power-of-two scales."""
    B, H, T, D, Bk, G = (cfg["batch"], cfg["kv_heads"], cfg["tokens"], cfg["head_dim"], cfg["k_block"],
                         cfg["v_group"])
    L = (1 << cfg["v_bits"]) - 1
    Lk = (1 << cfg["k_bits"]) - 1
    rng = np.random.default_rng(seed)
    v = np.empty((B, H, T, D))
    for g in range(D // G):
        s = 2.0 ** rng.integers(-3, 2, (B, H, T, 1))
        z = rng.integers(-8, 8, (B, H, T, 1)) * s
        k_half = rng.integers(0, L, (B, H, T, G)) + 0.5
        row = z + k_half * s
        row[..., 0:1] = z
        row[..., 1:2] = z + L * s
        v[..., g * G:(g + 1) * G] = row
    k = np.empty((B, H, T, D))
    for n in range((T + Bk - 1) // Bk):
        t0, t1 = n * Bk, min(T, (n + 1) * Bk)
        s = 2.0 ** rng.integers(-3, 2, (B, H, 1, D))
        z = rng.integers(-8, 8, (B, H, 1, D)) * s
        blk = z + (rng.integers(0, Lk, (B, H, t1 - t0, D)) + 0.5) * s
        blk[:, :, 0:1] = z
        if t1 - t0 > 1:
            blk[:, :, 1:2] = z + Lk * s
        k[:, :, t0:t1] = blk
    return f16(k), f16(v)


def constant_inputs(cfg, seed=6):
    """Constant value rows (one group constant, the next random) and key channels
    that are constant over every block; one channel per head 40x larger than the
    rest, so that with outliers on it is every token's top entry (an empty channel)."""
    B, H, T, D = cfg["batch"], cfg["kv_heads"], cfg["tokens"], cfg["head_dim"]
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((B, H, T, D))
    v[..., : cfg["v_group"]] = rng.integers(-4, 5, (B, H, T, 1)) * 0.75
    kc = rng.standard_normal((B, H, 1, D))
    k = np.repeat(kc, T, axis=2)
    k[..., D // 3] = 40.0 + rng.random((B, H, T))
    k[..., D // 2:] += rng.standard_normal((B, H, T, D - D // 2))   # half the channels vary
    return f16(k), f16(v)


EDGE = {
    "ties_plain": synth.config("c1", batch=1, q_heads=2, kv_heads=2, tokens=3 * 128 + 21, capacity=512),
    "ties_clip_csr": synth.config("c4", batch=1, q_heads=2, kv_heads=2, tokens=3 * 128 + 21, capacity=512,
                                  existing=0),
    "ties_d64_v2_g16": synth.config("c0", v_bits=2, v_group=16, tokens=4 * 64 + 9, capacity=320),
    "ties_gqa_csr": synth.config("c2", batch=1, q_heads=8, kv_heads=2, tokens=3 * 128 + 5, capacity=512,
                                 inject=False),
    "const_plain": synth.config("c1", batch=1, q_heads=2, kv_heads=2, v_group=64, tokens=2 * 128 + 40,
                                capacity=384),
    "const_clip_csr": synth.config("c4", batch=1, q_heads=2, kv_heads=2, v_group=64, tokens=2 * 128 + 40,
                                   capacity=384, existing=0),
    "const_gqa_csr": synth.config("c2", batch=1, q_heads=4, kv_heads=1, tokens=3 * 128, capacity=384,
                                  inject=False),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_degenerate_groups_bitwise(case):
    import oracle
    cfg = EDGE[case]
    say("case", case, cfg)
    k, v = (tie_inputs if case.startswith("ties") else constant_inputs)(cfg)
    T = cfg["tokens"]
    cache = build_gpu_cache(cfg, k, v, [T // 2, T - T // 2])
    heads = oracle_heads(cfg, k, v)
    ko = oracle.kout(cfg)
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, ko, b, h)
        if case.startswith("const"):
            assert (hc.v_scale[:, 0] == 0).sum() >= (T // cfg["k_block"]) * cfg["k_block"] - 1
    for which in (0, 1):
        g = cache.dequantize(which).cpu().numpy()
        for (b, h), hc in heads.items():
            assert np.array_equal(g[b, h].view(np.uint32), hc.dequantize(which).view(np.uint32)), (which, b, h)
    q = synth.gen_q(cfg)
    B, Hq, H = cfg["batch"], cfg["q_heads"], cfg["kv_heads"]
    gq = Hq // H
    out = cache.decode(upload(q), q_pos=T - 1).cpu().numpy().astype(np.float64)
    hl = [heads[(b, hq // gq)] for b in range(B) for hq in range(Hq)]
    ql = np.stack([q[b, hq] for b in range(B) for hq in range(Hq)])
    ref = oracle.decode_many(cfg, hl, ql, T - 1).reshape(B, Hq, -1)
    err = np.abs(out - ref).max()
    say("  decode max abs err", err)
    assert err <= TOL


def test_ties_hit_the_exact_branch():
    """The tie inputs really produce half-integer quotients (checked on the oracle's
    stored metadata): the scale is the power of two the row was built with."""
    cfg = EDGE["ties_plain"]
    k, v = tie_inputs(cfg)
    hc = oracle_heads(cfg, k, v, heads={(0, 0)})[(0, 0)]
    s = hc.v_scale[: (cfg["tokens"] // 128) * 128, 0].view(np.float16).astype(np.float64)
    assert np.all(np.log2(s) == np.round(np.log2(s)))


MANY = synth.config("c3", batch=1, q_heads=8, kv_heads=8, tokens=131072, capacity=131072)


@pytest.mark.timeout(600)
def test_decode_with_1024_and_4096_splits():
    import oracle
    cfg = MANY
    say("long-context codebook cache, 1024 blocks per head")
    lut = synth.calib_lut(cfg)
    k = synth.gen_tensor(cfg, synth.TENSOR_K)
    v = synth.gen_tensor(cfg, synth.TENSOR_V)
    cache = build_gpu_cache(cfg, k, v, [65536, 65536], lut)
    heads = {(0, h): hc for h, hc in enumerate(
        oracle.build_heads(cfg, k[0], v[0], [lut[h] for h in range(cfg["kv_heads"])]))}
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, 0, b, h)
    say("  caches bitwise equal")
    q = synth.gen_q(cfg)
    T, Hq = cfg["tokens"], cfg["q_heads"]
    ref = oracle.decode_many(cfg, [heads[(0, h)] for h in range(Hq)], q[0], T - 1)
    vmax = max(float(np.abs(hc.dequantize(1)).max()) for hc in heads.values())
    qd = upload(q)
    outs = {}
    for S in (0, 1024, 4096):
        a = cache.decode(qd, q_pos=T - 1, num_splits=S).cpu().numpy()
        b = cache.decode(qd, q_pos=T - 1, num_splits=S).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), S
        err = np.abs(a[0].astype(np.float64) - ref).max()
        say("  splits", S or "auto", "max abs err", err)
        assert err <= TOL
        outs[S] = a
    nblk = T // cfg["k_block"]
    for S in (1024, 4096):
        d = np.abs(outs[S] - outs[0]).max()
        say("  splits", S, "vs auto: max diff", d, "bound", split_tol(vmax, nblk, S, 64))
        assert d <= split_tol(vmax, nblk, S, 64)
