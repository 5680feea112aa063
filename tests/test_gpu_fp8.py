"""GPU parity of the FP8 cache (k_mode 2 with v_mode 2): keys and values cast to OCP
E4M3, nearest with ties to even, saturating at +-448.

Against the CPU oracle: the packed bytes bit for bit after ragged appends (inputs of
magnitude up to several hundred, past 448 and with fp16 subnormals, so that rounding
ties, saturation and the subnormal range are all reached); decode and chunk attention
within 2e-3; dequantized keys and values bit for bit; a paged pool; fused steps.
"""
import numpy as np
import pytest

import synth
from _gpu_util import build_gpu_cache, compare_head, inputs, say, upload

pytestmark = pytest.mark.gpu

TOL = 2e-3
FP8 = dict(k_mode=2, k_bits=8, v_mode=2, v_bits=8)


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
    "mha_d128": (synth.config("c1", batch=2, q_heads=2, kv_heads=2, tokens=5 * 128 + 50, capacity=768, **FP8),
                 [200, 1, 300, 189]),
    "gqa_d64": (synth.config("c0", q_heads=8, kv_heads=2, tokens=5 * 64 + 17, capacity=384, **FP8), [64, 100, 173]),
    "gqa_d128_bk64": (synth.config("c2", batch=1, q_heads=8, kv_heads=2, k_block=64, tokens=6 * 64 + 9,
                                   capacity=448, outlier_pct=0, inject=False, **FP8), None),
}


def _stress(k, v):
    """Spread the inputs over E4M3's range: large keys (some past 448), exact ties of
    the E4M3 grid, fp16 subnormals."""
    k = k.copy(); v = v.copy()
    kf = k.view(np.float16).astype(np.float32) * 37.0
    kf[..., ::17, 3] = 600.0
    kf[..., ::19, 5] = 1.0625                                # a tie: 1 + 1/16
    vf = v.view(np.float16).astype(np.float32)
    vf[..., ::13, 7] = 2.0 ** -20
    return kf.astype(np.float16).view(np.uint16), vf.astype(np.float16).view(np.uint16)


def _heads(cfg, k, v, lengths=None):
    import oracle
    out = {}
    for b in range(cfg["batch"]):
        L = cfg["tokens"] if lengths is None else lengths[b]
        for h in range(cfg["kv_heads"]):
            out[(b, h)] = oracle.HeadCache(dict(cfg, tokens=L)).build(k[b, h, :L], v[b, h, :L])
    return out


@pytest.mark.parametrize("case", sorted(CASES))
def test_fp8_cache_matches_oracle(case):
    import torch
    import oracle
    cfg, chunks = CASES[case]
    T, B, H, Hq = cfg["tokens"], cfg["batch"], cfg["kv_heads"], cfg["q_heads"]
    gq = Hq // H
    say("case", case)
    k, v = _stress(*inputs(cfg))
    cache = build_gpu_cache(cfg, k, v, chunks)
    heads = _heads(cfg, k, v)
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, 0, b, h)
    for which in (0, 1):
        g = cache.dequantize(which).cpu().numpy()
        for (b, h), hc in heads.items():
            assert np.array_equal(g[b, h].view(np.uint32), hc.dequantize(which).view(np.uint32)), (which, b, h)
    hl = [heads[(b, hq // gq)] for b in range(B) for hq in range(Hq)]
    q = synth.gen_q(cfg)
    q = (q.view(np.float16).astype(np.float32) * 0.03).astype(np.float16).view(np.uint16)   # scores of order 1
    qd = upload(q)
    for qp in (T - 1, T + 300, 7):
        for S in (0, 3):
            out = cache.decode(qd, q_pos=qp, num_splits=S).cpu().numpy().astype(np.float64)
            ref = oracle.decode_many(cfg, hl, q.reshape(B * Hq, -1), qp).reshape(out.shape)
            err = float(np.abs(out - ref).max())
            say("  decode q_pos", qp, "splits", S, "max abs err", err)
            assert err <= TOL
    nq = 7
    qc = (synth.gen_q_chunk(cfg, nq).view(np.float16).astype(np.float32) * 0.03).astype(np.float16).view(np.uint16)
    outc = cache.chunk(upload(qc), q_pos=T - nq - 40).cpu().numpy().astype(np.float64)
    refc = oracle.chunk_many(cfg, hl, qc.reshape(B * Hq, nq, -1), nq, T - nq - 40).reshape(outc.shape)
    errc = float(np.abs(outc - refc).max())
    say("  chunk max abs err", errc)
    assert errc <= TOL
    torch.cuda.synchronize()


def test_fp8_cache_in_a_paged_pool():
    import torch
    import oracle
    import quantized_decode_attn_amd as kvq
    cfg, _ = CASES["mha_d128"]
    B, H, Hq, Bk = cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["k_block"]
    k, v = _stress(*inputs(cfg))
    lengths = [cfg["tokens"], 3 * Bk + 1]
    need = [-(-L // Bk) for L in lengths]
    perm = np.random.default_rng(13).permutation(sum(need) + 2)
    table = np.full((B, cfg["capacity"] // Bk), 1 << 20, np.int32)
    table[0, :need[0]] = perm[:need[0]]
    table[1, :need[1]] = perm[need[0]:need[0] + need[1]]
    dev = torch.device("cuda:0")
    paged = kvq.PagedCache(cfg, num_blocks=len(perm), block_table=torch.from_numpy(table).to(dev), device=dev)
    paged.append_seqs(upload(k), upload(v), lengths)
    heads = _heads(cfg, k, v, lengths)
    q = (synth.gen_q(cfg).view(np.float16).astype(np.float32) * 0.03).astype(np.float16).view(np.uint16)
    out = paged.decode(upload(q)).cpu().numpy().astype(np.float64)
    gq = Hq // H
    for b in range(B):
        ref = oracle.decode_many(dict(cfg, tokens=lengths[b]), [heads[(b, hq // gq)] for hq in range(Hq)], q[b],
                                 lengths[b] - 1)
        err = float(np.abs(out[b] - ref).max())
        say("  sequence", b, "length", lengths[b], "max abs err", err)
        assert err <= TOL


def test_fp8_cache_in_fused_steps():
    import oracle
    cfg, _ = CASES["gqa_d64"]
    T, Bk = cfg["tokens"], cfg["k_block"]
    n_steps = T % Bk + 6
    T0 = T - n_steps
    H, Hq = cfg["kv_heads"], cfg["q_heads"]
    gq = Hq // H
    k, v = _stress(*inputs(cfg))
    cache = build_gpu_cache(cfg, k[:, :, :T0], v[:, :, :T0])
    qs = (synth.gen_q_chunk(cfg, n_steps).view(np.float16).astype(np.float32) * 0.03).astype(np.float16).view(np.uint16)
    kd, vd, qd = upload(k), upload(v), upload(qs)
    worst = 0.0
    for i in range(n_steps):
        t = T0 + i
        a = cache.step(kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), qd[:, :, i].contiguous())
        a = a.cpu().numpy().astype(np.float64)
        cfg_t = dict(cfg, tokens=t + 1)
        heads = _heads(cfg_t, k, v)
        ref = oracle.decode_many(cfg_t, [heads[(0, hq // gq)] for hq in range(Hq)], qs[0, :, i], t).reshape(a.shape)
        worst = max(worst, float(np.abs(a - ref).max()))
    say("  steps", n_steps, "max abs err", worst)
    assert worst <= TOL
    for (b, h), hc in _heads(cfg, k, v).items():
        compare_head(cache, hc, cfg, 0, b, h)


def test_fp8_nonfinite_inputs_cast_like_the_oracle():
    """NaN inputs stay NaN (S.1111.111, the cast's rare slow path) and infinities
    saturate to +-448, in keys and values: the bytes equal the oracle's and so do the
    dequantized bits."""
    import oracle
    cfg = synth.config("c0", tokens=3 * 64 + 5, capacity=256, **FP8)
    k, v = inputs(cfg)
    k = k.copy(); v = v.copy()
    k[0, 0, 3, 5] = 0x7E00; k[0, 1, 70, 0] = 0xFE01; k[0, 2, 130, 63] = 0x7C00; k[0, 3, 10, 9] = 0xFC00
    v[0, 0, 64, 1] = 0x7C00; v[0, 1, 65, 2] = 0xFE00; v[0, 3, 150, 40] = 0xFC00; v[0, 2, 5, 6] = 0x7E10
    cache = build_gpu_cache(cfg, k, v, [100, 97])
    heads = _heads(cfg, k, v)
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, 0, b, h)
    for which in (0, 1):
        g = cache.dequantize(which).cpu().numpy()
        for (b, h), hc in heads.items():
            assert np.array_equal(g[b, h].view(np.uint32), hc.dequantize(which).view(np.uint32)), (which, b, h)
