"""GPU parity under strongly peaked softmax (attention-sink-like inputs).

Every block holds one dominant key; the other keys are zero, so their softmax weights
sit 2^-17 .. 2^-20 below the dominant one (a different ratio in each block).  Value
rows span [-8, 8]: the small-weight tokens sit at the top code in all but one channel,
the dominant token at the bottom code.  A value contraction whose weights are rounded
relative to the block's largest weight (16-bit fixed point) is off by about 1e-2 here;
the decode output must stay within 2e-3 of the oracle on every element.

The inputs need no rotary arithmetic: the query and the dominant keys live on the
slowest rotary pair (channel D/2 - 1, angle below 0.1 rad over these lengths), so a
dominant key's score is a_g * b / sqrt(D) to within cos(0.1).
"""
import numpy as np
import pytest

import synth
from _gpu_util import build_gpu_cache, compare_head, oracle_heads, say, upload

pytestmark = pytest.mark.gpu

TOL = 2e-3
LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import quantized_decode_attn_amd as kvq
    kvq.lib()
    import oracle
    oracle.build()


def f16(x):
    return np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float16)).view(np.uint16)


def peaked_inputs(cfg, seed=3):
    """Keys, values and queries (fp16 bits) of the peaked workload described above."""
    B, H, Hq, D, T, Bk = (cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["head_dim"],
                          cfg["tokens"], cfg["k_block"])
    gq = Hq // H
    rng = np.random.default_rng(seed)
    ch = D // 2 - 1                                   # slowest rotary pair, component a
    a = 12.0 * (1.0 + 0.05 * np.arange(gq))          # query amplitude per head of a group
    k = np.zeros((B, H, T, D))
    v = np.full((B, H, T, D), 8.0)
    lowch = rng.integers(0, D, (B, H, T))            # the one channel at -8 in a small-weight row
    v[np.arange(B)[:, None, None], np.arange(H)[None, :, None], np.arange(T)[None, None, :], lowch] = -8.0
    nblk = (T + Bk - 1) // Bk
    for n in range(nblk):
        r = 17 + n % 4                               # log2 of the weight ratio, this block
        b = r * np.sqrt(D) / (LOG2E * a[0])          # dominant score of head 0: r * ln 2
        t = n * Bk + int(rng.integers(0, min(Bk, T - n * Bk)))
        k[:, :, t, ch] = b
        v[:, :, t, :] = -8.0
        v[:, :, t, (n * 7) % D] = 8.0
    q = np.zeros((B, Hq, D))
    for hq in range(Hq):
        q[:, hq, ch] = a[hq % gq]
    return f16(k), f16(v), f16(q)


CASES = {
    # one query head per kv head
    "mha_d64_bk64": synth.config("c0", batch=2, tokens=5 * 64 + 37, capacity=384),
    "mha_d128_bk128": synth.config("c1", batch=1, q_heads=3, kv_heads=3, tokens=5 * 128 + 37,
                                   capacity=768),
    "mha_d128_g64_csr": synth.config("c4", batch=1, q_heads=2, kv_heads=2, tokens=4 * 128 + 5,
                                     capacity=640, existing=0, clip_quantile=0.0),
    # grouped-query: 2, 4 and 8 query heads per kv head
    "gqa2": synth.config("c2", batch=1, q_heads=4, kv_heads=2, tokens=5 * 128 + 37, capacity=768,
                         inject=False),
    "gqa4": synth.config("c2", batch=1, q_heads=8, kv_heads=2, tokens=5 * 128 + 37, capacity=768,
                         inject=False),
    "gqa8_g64": synth.config("c2", batch=1, q_heads=8, kv_heads=1, v_group=64, tokens=6 * 128,
                             capacity=768, inject=False),
}
CASES["mha_d128_g64_csr"]["v_group"] = 64


@pytest.mark.parametrize("case", sorted(CASES))
def test_peaked_softmax(case):
    import oracle
    cfg = CASES[case]
    say("case", case, cfg)
    k, v, q = peaked_inputs(cfg)
    cache = build_gpu_cache(cfg, k, v, [cfg["tokens"] // 3, cfg["tokens"] - cfg["tokens"] // 3])
    heads = oracle_heads(cfg, k, v)
    ko = oracle.kout(cfg)
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, ko, b, h)
    B, Hq, H = cfg["batch"], cfg["q_heads"], cfg["kv_heads"]
    gq = Hq // H
    qd = upload(q)
    for S in (0, 1, 3):
        out = cache.decode(qd, q_pos=cfg["tokens"] - 1, num_splits=S).cpu().numpy().astype(np.float64)
        hl, ql = [], []
        for b in range(B):
            for hq in range(Hq):
                hl.append(heads[(b, hq // gq)])
                ql.append(q[b, hq])
        ref = oracle.decode_many(cfg, hl, np.stack(ql), cfg["tokens"] - 1).reshape(B, Hq, -1)
        err = np.abs(out - ref).max()
        say("  splits", S or "auto", "max abs err", err, "output range", float(np.abs(ref).max()))
        assert err <= TOL
