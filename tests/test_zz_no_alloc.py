"""kvq_decode_attention_noalloc against kvq_decode_attention, through the C ABI.

The no-allocation decode keeps its split partials in the library's per-GPU device
array instead of a caller workspace; for the same num_splits it must give bitwise the
output of the workspace decode (same kernels), and both must be within 2e-3 of the
oracle.  Two calls in a row, the second on a smaller cache, so the second reuses an
array that still holds the first call's partials.
"""
import numpy as np
import pytest

import synth
from _gpu_util import build_gpu_cache, inputs, oracle_heads, say, upload

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


CALLS = [
    ("large", synth.config("c4", batch=2, q_heads=4, kv_heads=4, tokens=6 * 128 + 50, capacity=896,
                           existing=0), 0),
    ("small", synth.config("c0", tokens=100, capacity=128), 3),
]


def _oracle_out(cfg, k, v, q):
    import oracle
    heads = oracle_heads(cfg, k, v)
    B, Hq, H = cfg["batch"], cfg["q_heads"], cfg["kv_heads"]
    gq = Hq // H
    hl = [heads[(b, hq // gq)] for b in range(B) for hq in range(Hq)]
    ql = np.stack([q[b, hq] for b in range(B) for hq in range(Hq)])
    return oracle.decode_many(cfg, hl, ql, cfg["tokens"] - 1).reshape(B, Hq, -1)


def test_noalloc_decode_matches_workspace_decode_twice():
    import torch
    import quantized_decode_attn_amd as kvq
    for name, cfg, S in CALLS:
        say("call", name, cfg["workload"], "tokens", cfg["tokens"], "splits", S or "auto")
        k, v = inputs(cfg)
        cache = build_gpu_cache(cfg, k, v)
        q = synth.gen_q(cfg)
        qd = upload(q)
        ref_ws = cache.decode(qd, q_pos=cfg["tokens"] - 1, num_splits=S)
        out = torch.full_like(ref_ws, float("nan"))
        kvq.kvq_decode_attention_noalloc(cache.desc, qd, cfg["tokens"] - 1, out, S)
        torch.cuda.synchronize()
        a = out.cpu().numpy()
        b = ref_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
        err = np.abs(a.astype(np.float64) - _oracle_out(cfg, k, v, q)).max()
        say("  bitwise equal to the workspace decode; max abs err vs oracle", err)
        assert err <= TOL


def test_noalloc_rejects_partials_beyond_its_array():
    import torch
    import quantized_decode_attn_amd as kvq
    cfg = synth.config("c0", tokens=100, capacity=128)
    k, v = inputs(cfg)
    cache = build_gpu_cache(cfg, k, v)
    q = upload(synth.gen_q(cfg))
    out = torch.empty((1, 4, 64), dtype=torch.float32, device="cuda")
    per_split = cfg["batch"] * cfg["q_heads"] * (cfg["head_dim"] + 2) * 4
    assert 4096 * per_split < kvq.NOALLOC_SCRATCH_BYTES        # this one fits ...
    kvq.kvq_decode_attention_noalloc(cache.desc, q, 99, out, 4096)
    big = synth.config("c1", tokens=128, capacity=128)           # ... B 8 x 32 heads x 4096 splits does not
    cache2 = build_gpu_cache(big, *inputs(big))
    out2 = torch.empty((8, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention_noalloc(cache2.desc, upload(synth.gen_q(big)), 127, out2, 4096)
    assert e.value.status == kvq.KVQ_EWORKSPACE
    torch.cuda.synchronize()
