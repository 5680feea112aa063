"""GPU parity of keys kept in fp16 by L2 norm (keep_pct > 0: in every quantized block the
ceil(p * k_block / 100) key vectors of largest squared L2 norm stay exact fp16 and leave
the block's statistics).

Against the CPU oracle: the cache buffers, the kept tokens' offsets and rows included,
bit for bit after appends in ragged chunks; decode and chunk attention within 2e-3 of
the oracle's fp64 attention (4-bit keys with one query head per kv head at head_dim 128
take the tuned kernel, which rescores the kept tokens from their fp16 rows; the rest take
the generic kernel, whose fp16 key path they share with the tail); dequantized keys bit for bit; a paged cache with kept keys;
and a planted key of huge norm, which only a kept fp16 copy reproduces.
"""
import numpy as np
import pytest

import synth
from _gpu_util import build_gpu_cache, compare_head, inputs, oracle_heads, say, upload

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
    # (config, append chunks)
    "mha_d128_keep7": (synth.config("c1", batch=2, q_heads=2, kv_heads=2, tokens=5 * 128 + 50, capacity=768,
                                    keep_pct=5), [200, 1, 300, 189]),
    "gqa_d64_keep8": (synth.config("c0", q_heads=8, kv_heads=2, v_bits=2, v_group=32, tokens=5 * 64 + 17,
                                   capacity=384, keep_pct=12), [64, 100, 173]),
    "mha_v2_keep13": (synth.config("c1", batch=1, q_heads=2, kv_heads=2, v_bits=2, v_group=64, tokens=4 * 128 + 77,
                                   capacity=640, keep_pct=10), [300, 289]),
    "k2_keep16": (synth.config("c1", batch=1, q_heads=2, kv_heads=2, k_bits=2, v_group=32, tokens=3 * 128 + 9,
                               capacity=512, keep_pct=12), None),
    "k3_keep2": (synth.config("c1", batch=1, q_heads=4, kv_heads=2, k_bits=3, tokens=4 * 128, capacity=512,
                              keep_pct=1), [128, 256, 128]),
}


def _planted(cfg, k):
    """A few keys of every block scaled far above the rest (large, off-grid norms)."""
    k = k.copy()
    Bk = cfg["k_block"]
    x = k.view(np.float16).astype(np.float32)
    for n in range(k.shape[2] // Bk):
        for j in (3, Bk // 2 + 1):
            x[:, :, n * Bk + j] = x[:, :, n * Bk + j] * 7.0 + 3.0
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("case", sorted(CASES))
def test_kept_keys_match_oracle(case):
    import torch
    import oracle
    cfg, chunks = CASES[case]
    T = cfg["tokens"]
    B, H, Hq = cfg["batch"], cfg["kv_heads"], cfg["q_heads"]
    gq = Hq // H
    k, v = inputs(cfg)
    k = _planted(cfg, k)
    cache = build_gpu_cache(cfg, k, v, chunks)
    heads = oracle_heads(cfg, k, v)
    say("case", case, "kept per block", oracle.keep_count(cfg))
    ko = oracle.kout(cfg)
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, ko, b, h)
    # decode at the newest token and past the end
    q = synth.gen_q(cfg)
    qd = upload(q)
    for qp in (T - 1, T + 500):
        out = cache.decode(qd, q_pos=qp).cpu().numpy().astype(np.float64)
        hl = [heads[(b, hq // gq)] for b in range(B) for hq in range(Hq)]
        ref = oracle.decode_many(cfg, hl, q.reshape(B * Hq, -1), qp).reshape(out.shape)
        err = float(np.abs(out - ref).max())
        say("  decode q_pos", qp, "max abs err", err)
        assert err <= TOL
    # a causal chunk reaching back over the quantized blocks
    nq = 9
    qc = synth.gen_q_chunk(cfg, nq)
    outc = cache.chunk(upload(qc), q_pos=T - nq - 70).cpu().numpy().astype(np.float64)
    hl = [heads[(b, hq // gq)] for b in range(B) for hq in range(Hq)]
    refc = oracle.chunk_many(cfg, hl, qc.reshape(B * Hq, nq, -1), nq, T - nq - 70).reshape(outc.shape)
    errc = float(np.abs(outc - refc).max())
    say("  chunk max abs err", errc)
    assert errc <= TOL
    # dequantized keys, bit for bit
    dk = cache.dequantize(0).cpu().numpy()
    for (b, h), hc in heads.items():
        assert np.array_equal(dk[b, h].view(np.uint32), hc.dequantize(0).view(np.uint32)), (b, h)
    torch.cuda.synchronize()


def test_kept_keys_in_a_paged_cache():
    """Kept keys live in the block's slot: a shuffled pool gives the oracle's decode."""
    import torch
    import oracle
    import quantized_decode_attn_amd as kvq
    cfg, _ = CASES["mha_d128_keep7"]
    cfg = dict(cfg)
    B, H, Hq, Bk = cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["k_block"]
    k, v = inputs(cfg)
    k = _planted(cfg, k)
    lengths = [cfg["tokens"], 3 * Bk + 5]
    need = [-(-L // Bk) for L in lengths]
    rng = np.random.default_rng(5)
    perm = rng.permutation(sum(need) + 2)
    table = np.full((B, cfg["capacity"] // Bk), 1 << 20, np.int32)
    table[0, :need[0]] = perm[:need[0]]
    table[1, :need[1]] = perm[need[0]:need[0] + need[1]]
    dev = torch.device("cuda:0")
    paged = kvq.PagedCache(cfg, num_blocks=len(perm), block_table=torch.from_numpy(table).to(dev), device=dev)
    paged.append_seqs(upload(k), upload(v), lengths)
    q = synth.gen_q(cfg)
    out = paged.decode(upload(q)).cpu().numpy().astype(np.float64)
    gq = Hq // H
    for b in range(B):
        L = lengths[b]
        hs = [oracle.HeadCache(cfg).build(k[b, h, :L], v[b, h, :L]) for h in range(H)]
        ref = oracle.decode_many(cfg, [hs[hq // gq] for hq in range(Hq)], q[b], L - 1)
        err = float(np.abs(out[b] - ref).max())
        say("  sequence", b, "length", L, "max abs err", err)
        assert err <= TOL


def test_norm_rounding_decides_the_kept_key():
    """Row A: 2048 in channel 0, then 63 channels of 2^-16; in channel order every
    tiny square (a quarter ulp of 2^22) rounds away and the norm is exactly 2^22.  Row
    B: 2048 and 2^-15, norm 2^22 + 2^-30 exactly.  With one key kept per block the
    oracle keeps B; a sum in another order (the tiny squares first) would make A the
    larger.  The kernel's parallel sum must fall back to channel order here."""
    import oracle
    cfg = synth.config("c0", batch=1, q_heads=2, kv_heads=2, k_block=64, tokens=3 * 64 + 5, capacity=256,
                       keep_pct=1)
    assert oracle.keep_count(cfg) == 1
    k, v = inputs(cfg)
    k = k.copy()
    for n in range(3):
        for h in range(2):
            a = np.full(64, 0x0100, np.uint16)      # 2^-16 (subnormal)
            a[0] = 0x6800                          # 2048
            bb = np.zeros(64, np.uint16)
            bb[0], bb[1] = 0x6800, 0x0200          # 2048, 2^-15
            ja, jb = (5, 40) if n != 1 else (40, 5)
            k[0, h, n * 64 + ja] = a
            k[0, h, n * 64 + jb] = bb
    cache = build_gpu_cache(cfg, k, v, [70, 127])
    heads = oracle_heads(cfg, k, v)
    for (b, h), hc in heads.items():
        assert list(hc.k_keep_idx[:3].reshape(-1)) == [40, 5, 40]
        compare_head(cache, hc, cfg, oracle.kout(cfg), b, h)
