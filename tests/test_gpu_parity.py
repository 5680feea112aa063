"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Quantized caches (codes, scales, zeros, outlier CSR, tails) and dequantized values
must be bit-identical; decode outputs must be within 2e-3 (max abs) of the oracle's
fp64 attention over the same quantized cache.  Small cases span several blocks and a
ragged tail and are compared in full; the five workloads at their full sizes are
compared on every head, in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

import synth
from _gpu_util import build_gpu_cache, compare_head, inputs, oracle_heads, say, upload

pytestmark = pytest.mark.gpu

TOL = 2e-3
U = 2.0 ** -24


def split_tol(vmax, nblk, s1, s2):
    """Largest difference between two decodes of one cache that differ only in their
    split counts s1, s2: each is an fp32 evaluation of the same normalised sum with at
    most nblk + s + 32 roundings (the blocks of a split, the merge, the cross-lane sums,
    the exponentials), each of relative size u = 2^-24 on terms bounded by max |v|."""
    return 4.0 * U * vmax * (nblk + s1 + s2 + 32)


def _vmax(cfg, k, v):
    """max |v| over the dequantized values (the oracle's), of every head."""
    import oracle
    heads = oracle_heads(cfg, k, v, _lut(cfg))
    return max(float(np.abs(hc.dequantize(1)).max()) for hc in heads.values())


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import quantized_decode_attn_amd as kvq
    kvq.lib()                                   # raises if the library is not built
    import oracle
    oracle.build()


SMALL = {
    "c0": (synth.config("c0"), None),
    "c0_ragged": (synth.config("c0", tokens=293, capacity=320), [37, 64, 192]),
    "mha_int4_d128": (synth.config("c1", batch=2, q_heads=4, kv_heads=4, tokens=3 * 128 + 50,
                                   capacity=512), [100, 30, 304]),
    "gqa_csr_inject": (synth.config("c2", batch=2, q_heads=8, kv_heads=2, tokens=4 * 128 + 77,
                                    capacity=640), None),
    "lut3_v2": (synth.config("c3", batch=1, q_heads=4, kv_heads=4, tokens=5 * 128 + 3,
                             capacity=768), [640, 3]),
    "clip_csr_append": (synth.config("c4", batch=2, q_heads=4, kv_heads=4, tokens=5 * 128 + 57,
                                     capacity=768), [2 * 128 + 17, 3 * 128 + 40]),
    "k2_v2_g16_gqa_d64": (synth.config("c0", k_bits=2, v_bits=2, v_group=16, tokens=200,
                                       capacity=256, q_heads=8, kv_heads=2), [5, 195]),
    "k3_uniform_g32": (synth.config("c1", batch=1, q_heads=2, kv_heads=2, k_bits=3, v_group=32,
                                    tokens=300, capacity=384), None),
    "lut4_bk64_csr": (synth.config("c3", batch=1, q_heads=2, kv_heads=2, k_bits=4, k_block=64,
                                   v_bits=4, v_group=128, tokens=333, capacity=384, outlier_pct=2),
                      None),
    "lut2_d64_clip": (synth.config("c0", k_mode=1, k_bits=2, v_group=32, tokens=150, capacity=192,
                                   clip_quantile=0.9), None),
    "lut3_v4_d64_bk64": (synth.config("c3", batch=2, q_heads=2, kv_heads=2, head_dim=64, k_block=64,
                                      v_bits=4, v_group=32, tokens=4 * 64 + 21, capacity=384),
                         [100, 177]),
    "lut2_v2_d128": (synth.config("c3", batch=1, q_heads=3, kv_heads=3, k_bits=2,
                                  tokens=3 * 128 + 9, capacity=512), None),
    # grouped-query: two heads per kv head (two of the four matrix rows carry zero weights)
    "gqa2_csr": (synth.config("c2", batch=1, q_heads=6, kv_heads=3, tokens=3 * 128 + 40,
                              capacity=512), None),
    # grouped-query: eight heads per kv head (two head sets), 2-bit values in groups of 64
    "gqa8_v2_g64": (synth.config("c2", batch=2, q_heads=16, kv_heads=2, v_bits=2, v_group=64,
                                 outlier_pct=0, inject=False, tokens=4 * 128 + 3, capacity=640),
                    [200, 315]),
    # grouped-query: 4-bit values in two groups of 64 channels, two outliers per vector
    "gqa4_v4_g64": (synth.config("c2", batch=1, q_heads=8, kv_heads=2, v_group=64,
                                 tokens=3 * 128 + 100, capacity=512), [128, 356]),
    # grouped-query: 2-bit values in one group of 128 channels, no outliers
    "gqa4_v2_g128": (synth.config("c2", batch=1, q_heads=4, kv_heads=1, v_bits=2, outlier_pct=0,
                                  inject=False, tokens=2 * 128 + 64, capacity=384), [100, 220]),
    # one head per kv head with one outlier per vector (head_dim 64: ceil(0.64) = 1)
    "mha_csr1_d64": (synth.config("c0", batch=2, outlier_pct=1, inject=True, tokens=5 * 64 + 30,
                                  capacity=384), [64, 286]),
    # the clip at the ends of its candidate path on a 128 x 128 tile: between the two
    # largest magnitudes (rank 1 from the top, the highest quantile below 1), the deepest
    # rank the candidate lists serve (255), and one rank deeper (256: the whole-tile
    # selection)
    "clip_rank1": (synth.config("c4", batch=1, q_heads=2, kv_heads=2, tokens=2 * 128 + 57, capacity=384,
                                existing=0, clip_quantile=(16383 - 1 + 0.5) / 16383), [128, 185]),
    "clip_rank255": (synth.config("c4", batch=1, q_heads=2, kv_heads=2, tokens=2 * 128 + 57,
                                  capacity=384, existing=0, clip_quantile=(16383 - 255 + 0.5) / 16383),
                     [128, 185]),
    "clip_rank256": (synth.config("c4", batch=1, q_heads=2, kv_heads=2, tokens=2 * 128 + 57,
                                  capacity=384, existing=0, clip_quantile=(16383 - 256 + 0.5) / 16383),
                     [128, 185]),
}


def _lut(cfg):
    return synth.calib_lut(cfg) if cfg["k_mode"] == 1 else None


def _q(cfg):
    return synth.gen_q(cfg)


def _decode_ref(cfg, heads, q, q_pos):
    """Oracle outputs [B][Hq][D] (fp64) for every (b, q-head)."""
    import oracle
    B, Hq, H = cfg["batch"], cfg["q_heads"], cfg["kv_heads"]
    gq = Hq // H
    hl, ql = [], []
    for b in range(B):
        for hq in range(Hq):
            hl.append(heads[(b, hq // gq)])
            ql.append(q[b, hq])
    out = oracle.decode_many(cfg, hl, np.stack(ql), q_pos)
    return out.reshape(B, Hq, -1)


@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_cases_bitwise_and_decode(case):
    import torch
    import oracle
    cfg, chunks = SMALL[case]
    say("case", case, cfg)
    k, v = inputs(cfg)
    lut = _lut(cfg)
    cache = build_gpu_cache(cfg, k, v, chunks, lut)
    heads = oracle_heads(cfg, k, v, lut)
    ko = oracle.kout(cfg)
    assert cache.length == cfg["tokens"]
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, ko, b, h)
    for which in (0, 1):
        g = cache.dequantize(which).cpu().numpy()
        for (b, h), hc in heads.items():
            o = hc.dequantize(which)
            assert np.array_equal(g[b, h].view(np.uint32), o.view(np.uint32)), (which, b, h)
    q = _q(cfg)
    qd = upload(q)
    for q_pos in (cfg["tokens"] - 1, cfg["tokens"] + 1000, 3):
        out = cache.decode(qd, q_pos=q_pos).cpu().numpy().astype(np.float64)
        ref = _decode_ref(cfg, heads, q, q_pos)
        err = np.abs(out - ref).max()
        say("  q_pos", q_pos, "max abs err", err)
        assert err <= TOL
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", ["clip_csr_append", "lut3_v2", "gqa_csr_inject"])
def test_split_count_invariance_and_determinism(case):
    cfg, _ = SMALL[case]
    say("case", case)
    k, v = inputs(cfg)
    cache = build_gpu_cache(cfg, k, v, None, _lut(cfg))
    qd = upload(_q(cfg))
    outs = {}
    for S in (1, 3, 7, 64):
        a = cache.decode(qd, num_splits=S).cpu().numpy()
        b = cache.decode(qd, num_splits=S).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), S
        outs[S] = a
    vmax = _vmax(cfg, k, v)
    nblk = cfg["tokens"] // cfg["k_block"]
    for S in (3, 7, 64):
        d = np.abs(outs[S] - outs[1]).max()
        say("  splits", S, "max diff vs 1 split", d, "bound", split_tol(vmax, nblk, 1, S))
        assert d <= split_tol(vmax, nblk, 1, S), S      # fp32 rounding order only


# Caches whose length is a whole number of blocks (no fp16 tail): the split merge then
# takes its one-round path for at most 16 splits and the LDS path above that.
NOTAIL = {
    "mha": synth.config("c1", batch=2, q_heads=4, kv_heads=4, tokens=20 * 128, capacity=20 * 128),
    "gqa_csr": synth.config("c2", batch=1, q_heads=8, kv_heads=2, tokens=12 * 128, capacity=12 * 128),
    "clip_csr": synth.config("c4", batch=1, q_heads=2, kv_heads=2, tokens=10 * 128, capacity=10 * 128,
                             existing=0),
}


@pytest.mark.parametrize("case", sorted(NOTAIL))
def test_merge_without_tail(case):
    cfg = NOTAIL[case]
    say("case", case)
    k, v = inputs(cfg)
    lut = _lut(cfg)
    cache = build_gpu_cache(cfg, k, v, None, lut)
    heads = oracle_heads(cfg, k, v, lut)
    q = _q(cfg)
    qd = upload(q)
    q_pos = cfg["tokens"] - 1
    ref = _decode_ref(cfg, heads, q, q_pos)
    nblk = cfg["tokens"] // cfg["k_block"]
    outs = {}
    # 16 and 17 straddle the one-round merge; nblk + 3 leaves some splits without a block
    for S in (1, 7, 16, 17, nblk + 3):
        a = cache.decode(qd, q_pos=q_pos, num_splits=S).cpu().numpy()
        b = cache.decode(qd, q_pos=q_pos, num_splits=S).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), S
        err = np.abs(a.astype(np.float64) - ref).max()
        say("  splits", S, "max abs err", err)
        assert err <= TOL, S
        outs[S] = a
    vmax = _vmax(cfg, k, v)
    for S in outs:
        assert np.abs(outs[S] - outs[1]).max() <= split_tol(vmax, nblk, 1, S), S   # fp32 rounding order only


@pytest.mark.parametrize("kind", ["equal_magnitudes", "few_levels"])
def test_clip_with_ties(kind):
    """The 99th-percentile clip and the outlier split when magnitudes repeat: every
    |x| equal (more candidates than the selection's lists hold, so the whole-tile
    selection runs), and values on a coarse grid (ties at the threshold and between
    outliers), compared bitwise with the oracle."""
    import oracle
    cfg, chunks = SMALL["clip_csr_append"]
    say("case", kind, cfg)
    k, v = inputs(cfg)
    rng = np.random.default_rng(7)
    f16 = lambda x: np.ascontiguousarray(x.astype(np.float16)).view(np.uint16)   # noqa: E731
    if kind == "equal_magnitudes":
        k = f16(np.where(rng.random(k.shape) < 0.5, -1.0, 1.0))
        v = f16(np.where(rng.random(v.shape) < 0.5, -0.75, 0.75))
    else:
        k = f16(np.round(k.view(np.float16).astype(np.float32) * 2.0) / 2.0)
        v = f16(np.round(v.view(np.float16).astype(np.float32) * 4.0) / 4.0)
    cache = build_gpu_cache(cfg, k, v, chunks)
    heads = oracle_heads(cfg, k, v)
    ko = oracle.kout(cfg)
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, ko, b, h)
    q = _q(cfg)
    out = cache.decode(upload(q)).cpu().numpy().astype(np.float64)
    ref = _decode_ref(cfg, heads, q, cfg["tokens"] - 1)
    assert np.abs(out - ref).max() <= TOL


@pytest.mark.parametrize("n", [1, 63, 64, 65])
def test_short_caches(n):
    """Tail-only caches, exactly one block, one block plus one token."""
    import oracle
    cfg = synth.config("c0", tokens=n, capacity=128)
    k, v = inputs(cfg)
    cache = build_gpu_cache(cfg, k, v, [n])
    heads = oracle_heads(cfg, k, v)
    for (b, h), hc in heads.items():
        compare_head(cache, hc, cfg, 0, b, h)
    q = _q(cfg)
    out = cache.decode(upload(q)).cpu().numpy()
    ref = _decode_ref(cfg, heads, q, n - 1)
    assert np.abs(out - ref).max() <= TOL


def test_append_errors_do_not_touch_the_cache():
    import quantized_decode_attn_amd as kvq
    cfg = synth.config("c0", tokens=100, capacity=128)
    k, v = inputs(cfg)
    cache = build_gpu_cache(cfg, k, v)
    before = {n: t.clone() for n, t in cache.bufs.items()}
    with pytest.raises(kvq.KvqError) as e:
        cache.append(upload(k[:, :, :29]), upload(v[:, :, :29]))
    assert e.value.status == kvq.KVQ_ECAPACITY and cache.length == 100
    for n, t in cache.bufs.items():
        assert bool((t == before[n]).all()), n


# --------------------------------------------------------------------------- full sizes
def _host_buffers(cache, cfg):
    """Every device buffer of the cache, copied to the host once."""
    return {n: t.cpu().numpy() for n, t in cache.bufs.items() if n not in ("rope", "k_lut")}


def _compare_head_host(bufs, hc, cfg, ko, b, h):
    from _gpu_util import defined_bytes, oracle_head_bytes, per_head_bytes
    bh = b * cfg["kv_heads"] + h
    per = per_head_bytes(cfg, ko)
    for name, nb in defined_bytes(cfg, ko, hc.length).items():
        if nb == 0:
            continue
        g = bufs[name][bh * per[name]: bh * per[name] + nb]
        o = oracle_head_bytes(hc, name, nb)
        if not np.array_equal(g, o):
            bad = np.nonzero(g != o)[0]
            raise AssertionError("%s differs at (b=%d, h=%d): %d of %d bytes, first at byte %d"
                                 % (name, b, h, bad.size, nb, bad[0]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_full_size_all_heads(name):
    """The workload at its full size, appended as the benchmark appends it (the prefill
    workload: its cached half, then the appended half), decoded in the launch
    configuration the benchmark times; every head's cache compared bitwise with the
    oracle and every (b, q-head) output within 2e-3 of the oracle's fp64 attention.
    The chunk attention the benchmark times with --chunk (16 queries at the newest
    positions, 4 on the 1M-token cache; automatic splits) is checked on the query heads
    of the first kv head."""
    import torch
    import oracle
    cfg = synth.config(name)
    say("full-size", name, cfg["workload"])
    lut = _lut(cfg)
    T, B, H, Hq = cfg["tokens"], cfg["batch"], cfg["kv_heads"], cfg["q_heads"]
    gq = Hq // H
    import quantized_decode_attn_amd as kvq
    dev = torch.device("cuda:0")
    lut_t = None if lut is None else torch.from_numpy(lut.view(np.int16)).to(dev)
    cache = kvq.Cache(cfg, device=dev, lut=lut_t)
    step = cfg["existing"] if cfg["existing"] else min(T, 131072)
    t = 0
    while t < T:
        n = min(step, T - t)
        k, v = inputs(cfg, t, t + n)
        cache.append(upload(k), upload(v))
        del k, v
        t += n
        say("  appended tokens", t, "of", T)
    q = synth.gen_q(cfg)
    out = cache.decode(upload(q)).cpu().numpy()
    nq = 4 if T > 500000 else 16
    qc = synth.gen_q_chunk(cfg, nq)
    outc = cache.chunk(upload(qc), q_pos=T - nq).cpu().numpy()
    torch.cuda.synchronize()
    bufs = _host_buffers(cache, cfg)
    ko = oracle.kout(cfg)
    # heads in batches of about 2 GiB of fp16 source per tensor
    per_batch = max(1, (1 << 30) // (T * cfg["head_dim"]))
    pairs = [(b, h) for b in range(B) for h in range(H)]
    worst = 0.0
    for i0 in range(0, len(pairs), per_batch):
        sel = pairs[i0:i0 + per_batch]
        kh = synth.gen_tensor(cfg, synth.TENSOR_K, heads=sel)
        vh = synth.gen_tensor(cfg, synth.TENSOR_V, heads=sel)
        hcs = oracle.build_heads(cfg, kh, vh, None if lut is None else [lut[h] for (_, h) in sel])
        del kh, vh
        for (b, h), hc in zip(sel, hcs):
            _compare_head_host(bufs, hc, cfg, ko, b, h)
        hl = [hc for hc in hcs for _ in range(gq)]
        ql = np.stack([q[b, h * gq + g] for (b, h) in sel for g in range(gq)])
        ref = oracle.decode_many(cfg, hl, ql, T - 1)
        got = np.stack([out[b, h * gq + g] for (b, h) in sel for g in range(gq)]).astype(np.float64)
        worst = max(worst, float(np.abs(got - ref).max()))
        if i0 == 0:   # chunk attention on the first kv head
            csel = sel[:1]
            hlc = [hc for hc in hcs[:1] for _ in range(gq)]
            qlc = np.stack([qc[b, h * gq + g] for (b, h) in csel for g in range(gq)])
            refc = oracle.chunk_many(cfg, hlc, qlc, nq, T - nq)
            gotc = np.stack([outc[b, h * gq + g] for (b, h) in csel for g in range(gq)]).astype(np.float64)
            errc = float(np.abs(gotc - refc).max())
            say("  chunk of", nq, "on", len(csel), "kv heads: max abs err", errc)
            assert errc <= TOL
        say("  heads", i0 + len(sel), "of", len(pairs), "bitwise equal; decode max abs err so far", worst)
        del hcs, hl
    assert worst <= TOL


def test_binding_rejects_mislaid_tensors():
    """The binding checks shape, dtype, contiguity and device before calling the C ABI."""
    import torch
    cfg = synth.config("c0", tokens=100, capacity=128)
    k, v = inputs(cfg)
    cache = build_gpu_cache(cfg, k, v)
    kd, vd = upload(k), upload(v)
    for bad in (kd[:, :2], kd.float(), kd.transpose(2, 3).contiguous().transpose(2, 3), kd.cpu()):
        with pytest.raises(ValueError):
            cache.append(bad, vd)
    q = upload(synth.gen_q(cfg))
    for bad in (q[:, :2], q.float(), q.transpose(1, 2).contiguous().transpose(1, 2)):
        with pytest.raises(ValueError):
            cache.decode(bad)
    with pytest.raises(ValueError):
        cache.decode(q, out=torch.empty((1, 4, 64), dtype=torch.float16, device="cuda"))
    assert cache.length == 100
