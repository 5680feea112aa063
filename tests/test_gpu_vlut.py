"""GPU parity of values quantized by a per-channel codebook (v_mode 1): a calibrated
(k-means) codebook and a log-spaced one (levels +-s 2^-k, the log quantization the
pages list among the non-uniform schemes).

Against the CPU oracle: the packed cache bit for bit after ragged appends; decode and
chunk attention within 2e-3 of the oracle's fp64 attention (the tuned one-head kernel
for 4-bit keys at head_dim 128, the generic kernel otherwise; both read each code's
entry from its channel's codebook); dequantized keys and values bit
for bit; a paged pool with ragged lengths; fused decode steps across a block boundary.
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
    # (config, value codebook kind, append chunks)
    "mha_d128_v4_log": (synth.config("c1", batch=2, q_heads=2, kv_heads=2, tokens=5 * 128 + 50, capacity=768,
                                     v_mode=1), "log", [200, 1, 300, 189]),
    "gqa_d64_v2_kmeans": (synth.config("c0", q_heads=8, kv_heads=2, v_bits=2, v_group=32, tokens=5 * 64 + 17,
                                       capacity=384, v_mode=1), "kmeans", [64, 100, 173]),
    "mha_d128_v2_kmeans": (synth.config("c1", batch=1, q_heads=3, kv_heads=3, v_bits=2, v_group=64,
                                        tokens=4 * 128 + 99, capacity=640, v_mode=1), "kmeans", [128, 300, 183]),
    "k3lut_v2_kmeans": (synth.config("c3", batch=1, q_heads=4, kv_heads=4, tokens=3 * 128 + 9, capacity=512,
                                     v_mode=1), "kmeans", None),
    "keep_and_v4_log": (synth.config("c1", batch=1, q_heads=2, kv_heads=2, tokens=4 * 128 + 77, capacity=640,
                                     keep_pct=5, v_mode=1), "log", [300, 289]),
}


def _books(cfg, kind):
    lut = synth.calib_lut(cfg) if cfg["k_mode"] == 1 else None
    vlut = synth.calib_log_vlut(cfg) if kind == "log" else synth.calib_vlut(cfg)
    return lut, vlut


def _heads(cfg, k, v, lut, vlut, lengths=None):
    import oracle
    out = {}
    for b in range(cfg["batch"]):
        L = cfg["tokens"] if lengths is None else lengths[b]
        for h in range(cfg["kv_heads"]):
            out[(b, h)] = oracle.HeadCache(dict(cfg, tokens=L), None if lut is None else lut[h], vlut[h]).build(
                k[b, h, :L], v[b, h, :L])
    return out


@pytest.mark.parametrize("case", sorted(CASES))
def test_codebook_values_match_oracle(case):
    import torch
    import oracle
    cfg, kind, chunks = CASES[case]
    T, B, H, Hq = cfg["tokens"], cfg["batch"], cfg["kv_heads"], cfg["q_heads"]
    gq = Hq // H
    say("case", case, kind)
    k, v = inputs(cfg)
    lut, vlut = _books(cfg, kind)
    cache = build_gpu_cache(cfg, k, v, chunks, lut, vlut)
    heads = _heads(cfg, k, v, lut, vlut)
    ko = oracle.kout(cfg)
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, ko, b, h)
    for which in (0, 1):
        g = cache.dequantize(which).cpu().numpy()
        for (b, h), hc in heads.items():
            assert np.array_equal(g[b, h].view(np.uint32), hc.dequantize(which).view(np.uint32)), (which, b, h)
    hl = [heads[(b, hq // gq)] for b in range(B) for hq in range(Hq)]
    q = synth.gen_q(cfg)
    qd = upload(q)
    for qp in (T - 1, T + 300, 7):
        for S in (0, 3):
            out = cache.decode(qd, q_pos=qp, num_splits=S).cpu().numpy().astype(np.float64)
            ref = oracle.decode_many(cfg, hl, q.reshape(B * Hq, -1), qp).reshape(out.shape)
            err = float(np.abs(out - ref).max())
            say("  decode q_pos", qp, "splits", S, "max abs err", err)
            assert err <= TOL
    nq = 7
    qc = synth.gen_q_chunk(cfg, nq)
    outc = cache.chunk(upload(qc), q_pos=T - nq - 40).cpu().numpy().astype(np.float64)
    refc = oracle.chunk_many(cfg, hl, qc.reshape(B * Hq, nq, -1), nq, T - nq - 40).reshape(outc.shape)
    errc = float(np.abs(outc - refc).max())
    say("  chunk max abs err", errc)
    assert errc <= TOL
    torch.cuda.synchronize()


def test_codebook_values_in_a_paged_pool():
    import torch
    import oracle
    import quantized_decode_attn_amd as kvq
    cfg, kind, _ = CASES["mha_d128_v4_log"]
    B, H, Hq, Bk = cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["k_block"]
    k, v = inputs(cfg)
    lut, vlut = _books(cfg, kind)
    lengths = [cfg["tokens"], 2 * Bk + 31]
    need = [-(-L // Bk) for L in lengths]
    perm = np.random.default_rng(9).permutation(sum(need) + 3)
    table = np.full((B, cfg["capacity"] // Bk), 1 << 20, np.int32)
    table[0, :need[0]] = perm[:need[0]]
    table[1, :need[1]] = perm[need[0]:need[0] + need[1]]
    dev = torch.device("cuda:0")
    paged = kvq.PagedCache(cfg, num_blocks=len(perm), block_table=torch.from_numpy(table).to(dev), device=dev,
                           vlut=torch.from_numpy(vlut.view(np.int16)).to(dev))
    half = [L // 2 for L in lengths]
    paged.append_seqs(upload(k), upload(v), half)
    rest_k = np.zeros_like(k)
    rest_v = np.zeros_like(v)
    for b in range(B):
        n = lengths[b] - half[b]
        rest_k[b, :, :n] = k[b, :, half[b]:lengths[b]]
        rest_v[b, :, :n] = v[b, :, half[b]:lengths[b]]
    paged.append_seqs(upload(rest_k), upload(rest_v), [lengths[b] - half[b] for b in range(B)])
    assert paged.lengths == lengths
    heads = _heads(cfg, k, v, lut, vlut, lengths)
    q = synth.gen_q(cfg)
    out = paged.decode(upload(q)).cpu().numpy().astype(np.float64)
    gq = Hq // H
    for b in range(B):
        ref = oracle.decode_many(dict(cfg, tokens=lengths[b]), [heads[(b, hq // gq)] for hq in range(Hq)], q[b],
                                 lengths[b] - 1)
        err = float(np.abs(out[b] - ref).max())
        say("  sequence", b, "length", lengths[b], "max abs err", err)
        assert err <= TOL


@pytest.mark.parametrize("case", ["gqa_d64_v2_kmeans", "mha_d128_v4_log"])
def test_codebook_values_in_fused_steps(case):
    """Token-by-token steps across a block boundary: the completed block is quantized
    with the codebook, and every step's output matches the oracle's decode over the
    tokens so far."""
    import oracle
    cfg, kind, _ = CASES[case]
    cfg = dict(cfg, batch=1)
    T = cfg["tokens"]
    Bk = cfg["k_block"]
    n_steps = T % Bk + 6                                  # crosses the last block boundary
    T0 = T - n_steps
    B, H, Hq = cfg["batch"], cfg["kv_heads"], cfg["q_heads"]
    gq = Hq // H
    k, v = inputs(cfg)
    lut, vlut = _books(cfg, kind)
    cache = build_gpu_cache(cfg, k[:, :, :T0], v[:, :, :T0], None, lut, vlut)
    qs = synth.gen_q_chunk(cfg, n_steps)
    kd, vd, qd = upload(k), upload(v), upload(qs)
    worst = 0.0
    for i in range(n_steps):
        t = T0 + i
        a = cache.step(kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), qd[:, :, i].contiguous())
        a = a.cpu().numpy().astype(np.float64)
        cfg_t = dict(cfg, tokens=t + 1)
        heads = _heads(cfg_t, k, v, lut, vlut)
        hl = [heads[(0, hq // gq)] for hq in range(Hq)]
        ref = oracle.decode_many(cfg_t, hl, qs[0, :, i], t).reshape(a.shape)
        worst = max(worst, float(np.abs(a - ref).max()))
    say("  steps", n_steps, "max abs err", worst)
    assert worst <= TOL
    ko = oracle.kout(cfg)
    for (b, h), hc in _heads(cfg, k, v, lut, vlut).items():
        compare_head(cache, hc, cfg, ko, b, h)
