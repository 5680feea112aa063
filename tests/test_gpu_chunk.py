"""GPU parity of causal chunk attention (several query tokens per sequence, query j at
position q_pos + j seeing the cache tokens t <= q_pos + j) against the CPU oracle's fp64
chunk attention over the same quantized cache: max abs error <= 2e-3.

Cases cover the matrix-core kernel (uniform 4-bit keys, head_dim 128, 128-token blocks;
one head and four heads per kv head, 2- and 4-bit values, one and two value groups,
none or two outliers per vector, clipping) and the generic kernel (codebook keys,
head_dim 64, 64-token blocks, one outlier per vector); chunks that end at the newest
token, that reach back over quantized blocks and the fp16 tail, that lie past the end or
start at position 0; row tiles of 16 with a ragged last tile; and several split counts.
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
    kvq.lib()                                   # raises if the library is not built
    import oracle
    oracle.build()


CASES = {
    # matrix-core kernel
    "mfma_mha_v4": (synth.config("c1", batch=2, q_heads=2, kv_heads=2, tokens=5 * 128 + 50,
                                 capacity=768), [300, 390]),
    "mfma_gqa4_v2_g64": (synth.config("c2", batch=1, q_heads=8, kv_heads=2, v_bits=2, v_group=64,
                                      outlier_pct=0, inject=False, tokens=4 * 128 + 77, capacity=640),
                         None),
    "mfma_mha_v2_notail": (synth.config("c1", batch=1, q_heads=2, kv_heads=2, v_bits=2, tokens=4 * 128,
                                        capacity=512), None),
    "mfma_gqa4_v4_g64": (synth.config("c2", batch=1, q_heads=4, kv_heads=1, v_group=64, outlier_pct=0,
                                      inject=False, tokens=6 * 128 + 5, capacity=896), None),
    "mfma_csr_gqa": (synth.config("c2", batch=1, q_heads=8, kv_heads=2, tokens=3 * 128 + 40,
                                  capacity=512), None),
    "mfma_clip_csr": (synth.config("c4", batch=1, q_heads=2, kv_heads=2, tokens=3 * 128 + 57,
                                   capacity=512), None),
    "mfma_csr_v2_g64": (synth.config("c2", batch=1, q_heads=4, kv_heads=1, v_bits=2, v_group=64,
                                     tokens=5 * 128 + 11, capacity=768), [200, 451]),
    # generic kernel
    "generic_csr1_d64": (synth.config("c0", batch=2, outlier_pct=1, inject=True, tokens=5 * 64 + 30,
                                      capacity=384), [64, 286]),
    "generic_lut3": (synth.config("c3", batch=1, q_heads=2, kv_heads=2, tokens=4 * 128 + 3,
                                  capacity=640), None),
    "generic_d64": (synth.config("c0", tokens=293, capacity=320), [37, 256]),
}


def _lut(cfg):
    return synth.calib_lut(cfg) if cfg["k_mode"] == 1 else None


def chunk_ref(cfg, heads, q, q_pos):
    """Oracle outputs [B][Hq][nq][D] (fp64) for every (b, q-head)."""
    import oracle
    B, Hq, H = cfg["batch"], cfg["q_heads"], cfg["kv_heads"]
    gq, nq = Hq // H, q.shape[2]
    hl, ql = [], []
    for b in range(B):
        for hq in range(Hq):
            hl.append(heads[(b, hq // gq)])
            ql.append(q[b, hq])
    out = oracle.chunk_many(cfg, hl, np.stack(ql), nq, q_pos)
    return out.reshape(B, Hq, nq, -1)


@pytest.mark.parametrize("case", sorted(CASES))
def test_chunk_matches_oracle(case):
    import torch
    cfg, chunks = CASES[case]
    T = cfg["tokens"]
    say("case", case, cfg)
    k, v = inputs(cfg)
    lut = _lut(cfg)
    cache = build_gpu_cache(cfg, k, v, chunks, lut)
    heads = oracle_heads(cfg, k, v, lut)
    # (nq, q_pos): the newest tokens, a chunk reaching back over quantized blocks, a
    # ragged 16-row tile, past the end, from position 0
    for nq, q_pos in ((5, T - 5), (37, T - 37), (16, T - 140), (3, T + 10), (4, 0)):
        q = synth.gen_q_chunk(cfg, nq)
        out = cache.chunk(upload(q), q_pos=q_pos).cpu().numpy().astype(np.float64)
        ref = chunk_ref(cfg, heads, q, q_pos)
        err = np.abs(out - ref).max()
        say("  nq", nq, "q_pos", q_pos, "max abs err", err)
        assert err <= TOL, (nq, q_pos)
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", ["mfma_mha_v4", "mfma_gqa4_v2_g64", "mfma_csr_gqa", "generic_csr1_d64"])
def test_chunk_split_counts_and_determinism(case):
    cfg, chunks = CASES[case]
    T = cfg["tokens"]
    say("case", case)
    k, v = inputs(cfg)
    lut = _lut(cfg)
    cache = build_gpu_cache(cfg, k, v, chunks, lut)
    heads = oracle_heads(cfg, k, v, lut)
    nq = 9
    q = synth.gen_q_chunk(cfg, nq)
    qd = upload(q)
    ref = chunk_ref(cfg, heads, q, T - nq)
    nblk = T // cfg["k_block"]
    for S in (1, 3, 4, 5, nblk, nblk + 3):
        a = cache.chunk(qd, num_splits=S).cpu().numpy()
        b = cache.chunk(qd, num_splits=S).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), S      # bitwise repeatable
        err = np.abs(a.astype(np.float64) - ref).max()
        say("  splits", S, "max abs err", err)
        assert err <= TOL, S


@pytest.mark.parametrize("case", ["mfma_mha_v4", "mfma_csr_gqa", "generic_csr1_d64"])
def test_chunk_of_one_is_the_decode_step(case):
    """nq = 1 at the newest position is single-query decode (both against the oracle,
    and against each other within fp32 rounding)."""
    cfg, chunks = CASES[case]
    T = cfg["tokens"]
    k, v = inputs(cfg)
    lut = _lut(cfg)
    cache = build_gpu_cache(cfg, k, v, chunks, lut)
    q = synth.gen_q_chunk(cfg, 1)
    qd = upload(q)
    a = cache.chunk(qd).cpu().numpy()[:, :, 0]
    d = cache.decode(qd[:, :, 0].contiguous(), q_pos=T - 1).cpu().numpy()
    heads = oracle_heads(cfg, k, v, lut)
    ref = chunk_ref(cfg, heads, q, T - 1)[:, :, 0]
    say("case", case, "chunk err", np.abs(a - ref).max(), "decode err", np.abs(d - ref).max())
    assert np.abs(a - ref).max() <= TOL and np.abs(d - ref).max() <= TOL
    assert np.abs(a - d).max() <= 1e-4


def test_chunk_binding_checks():
    import torch
    cfg, chunks = CASES["generic_d64"]
    k, v = inputs(cfg)
    cache = build_gpu_cache(cfg, k, v, chunks)
    q = upload(synth.gen_q_chunk(cfg, 4))
    for bad in (q[:, :2], q.float(), q.transpose(2, 3).contiguous().transpose(2, 3), q.cpu(), q[:, :, 0]):
        with pytest.raises(ValueError):
            cache.chunk(bad)
    import quantized_decode_attn_amd as kvq
    with pytest.raises(kvq.KvqError):
        cache.chunk(q, q_pos=-1)
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", ["mfma_mha_v4", "mfma_csr_gqa"])
def test_chunk_one_dominant_token(case):
    """One early token with a huge key component dominates the softmax of the rows that
    weigh it positively: every later block's probabilities fall below 2^-100 of it.  The
    per-block weight scaling must not overflow the accumulator for those rows (and the
    others, which give that token ~0 weight, must stay exact)."""
    cfg, chunks = CASES[case]
    T = cfg["tokens"]
    k, v = inputs(cfg)
    k = k.copy()
    k[:, :, 5, 3] = np.float16(30000.0).view(np.uint16)        # a dense value (c1) or the outlier (c2)
    lut = _lut(cfg)
    cache = build_gpu_cache(cfg, k, v, chunks, lut)
    heads = oracle_heads(cfg, k, v, lut)
    nq = 16
    q = synth.gen_q_chunk(cfg, nq)
    out = cache.chunk(upload(q), q_pos=T - nq).cpu().numpy().astype(np.float64)
    ref = chunk_ref(cfg, heads, q, T - nq)
    assert np.isfinite(out).all()
    err = np.abs(out - ref).max()
    say("case", case, "dominant token: max abs err", err)
    assert err <= TOL
