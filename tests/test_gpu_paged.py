"""GPU parity of caches with per-sequence lengths: the paged layout (quantized blocks in a
pool of physical blocks, each sequence's logical blocks mapped through a block table)
and the dense slots with per-sequence lengths, filled by ragged appends (each sequence
its own count per call: prefill chunks, single decode tokens, none) and decoded with
every sequence at its own newest position.

Against the CPU oracle, which knows nothing of paging: every sequence's decode output
within 2e-3 of the oracle's fp64 decode of a cache built from that sequence's tokens
alone, and every quantized block the sequence holds (read from the pool through the
table) and its fp16 tail equal to the oracle's bit for bit.  The paged cache and the
dense per-sequence cache give bitwise the same outputs (the same kernels; only the
block addressing differs); a plain dense cache at equal lengths gives the same outputs
within the split-order bound of fp32 (the per-sequence kernels choose each sequence's
split count by its length, so they may group the blocks differently).

Cases: the tuned one-head kernels (uniform 4-bit keys with 0 and 2 outliers per vector
and clipping; 3-bit codebook keys with 2-bit values), the tuned grouped-query kernel
(with outliers), and the generic kernel (head_dim 64 with grouped queries).
"""
import numpy as np
import pytest

import synth
from _gpu_util import say, upload

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


# (config, per-step counts [steps][batch]); the final lengths are the column sums
CASES = {
    "mha_v4": (synth.config("c1", batch=3, q_heads=2, kv_heads=2, tokens=1024, capacity=1024),
               [[300, 1, 77], [300, 1, 0], [0, 1, 77], [4, 129, 77], [23, 1, 1]]),
    "mha_csr_clip": (synth.config("c4", batch=3, q_heads=2, kv_heads=2, tokens=768, capacity=768, existing=0),
                     [[256, 5, 130], [1, 1, 1], [300, 0, 127], [211, 1, 0]]),
    "gqa_csr": (synth.config("c2", batch=2, q_heads=8, kv_heads=2, tokens=896, capacity=896),
                [[400, 128], [1, 1], [0, 300], [95, 1]]),
    "lut_v2": (synth.config("c3", batch=2, q_heads=2, kv_heads=2, tokens=640, capacity=640),
                    [[200, 3], [200, 129], [1, 0]]),
    "generic_gqa_d64": (synth.config("c0", batch=3, q_heads=8, kv_heads=2, tokens=512, capacity=512),
                        [[64, 3, 100], [1, 64, 100], [130, 0, 1]]),
}


def _lut(cfg):
    return synth.calib_lut(cfg) if cfg["k_mode"] == 1 else None


def _table(cfg, lengths, rng):
    """A shuffled pool: every block the sequences will hold gets its own physical block,
    in random order, with spare blocks; unused entries hold an out-of-pool value."""
    Bk, nb = cfg["k_block"], cfg["capacity"] // cfg["k_block"]
    need = [-(-L // Bk) for L in lengths]
    total = sum(need) + 3
    perm = rng.permutation(total)
    table = np.full((cfg["batch"], nb), 1 << 20, np.int32)
    i = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[i:i + n]
        i += n
    return table, total


def _oracle_decode(cfg, k, v, lut, lengths, q):
    """fp64 oracle outputs [B][Hq][D], each sequence from its own tokens and position."""
    import oracle
    B, H, Hq = cfg["batch"], cfg["kv_heads"], cfg["q_heads"]
    gq = Hq // H
    out = np.zeros((B, Hq, cfg["head_dim"]))
    heads = {}
    for b in range(B):
        L = lengths[b]
        for h in range(H):
            heads[(b, h)] = oracle.HeadCache(cfg, None if lut is None else lut[h]).build(k[b, h, :L], v[b, h, :L])
        hl = [heads[(b, hq // gq)] for hq in range(Hq)]
        out[b] = oracle.decode_many(cfg, hl, np.ascontiguousarray(q[b]), L - 1)
    return out, heads


def _slot_bytes(cfg, ko):
    D, Bk = cfg["head_dim"], cfg["k_block"]
    ng = D // cfg["v_group"]
    uni = cfg["k_mode"] == 0
    return {"k_codes": Bk * D * cfg["k_bits"] // 8, "k_scale": D * 2 if uni else 0, "k_zero": D * 2 if uni else 0,
            "v_codes": Bk * D * cfg["v_bits"] // 8, "v_scale": Bk * ng * 2, "v_zero": Bk * ng * 2,
            "k_col": Bk * ko, "k_val": Bk * ko * 2, "v_col": Bk * ko, "v_val": Bk * ko * 2}


def _compare_blocks(cache, table, cfg, ko, heads, lengths):
    """Every quantized block of every (b, h), read from its slot, against the oracle's
    block; the slot's row pointers; the fp16 tails."""
    H, Bk, D = cfg["kv_heads"], cfg["k_block"], cfg["head_dim"]
    per = _slot_bytes(cfg, ko)
    bufs = {name: cache.buffer(name).cpu().numpy() for name in per if per[name]}
    rp = {name: cache.buffer(name).cpu().numpy().view(np.int32) for name in ("k_rowptr", "v_rowptr") if ko}
    tails = {name: cache.buffer(name).cpu().numpy() for name in ("k_tail", "v_tail")}
    for (b, h), hc in heads.items():
        L = lengths[b]
        for n in range(L // Bk):
            g = (int(table[b, n]) * H + h) if table is not None else ((b * H + h) * (cfg["capacity"] // Bk) + n)
            for name, nb in per.items():
                if nb == 0:
                    continue
                gpu = bufs[name][g * nb:(g + 1) * nb]
                ora = np.ascontiguousarray(getattr(hc, name)).view(np.uint8).reshape(-1)[n * nb:(n + 1) * nb]
                assert np.array_equal(gpu, ora), (name, b, h, n)
            if ko and table is not None:
                for name in rp:
                    assert np.array_equal(rp[name][g * (Bk + 1):(g + 1) * (Bk + 1)], np.arange(Bk + 1) * ko), (name, b, n)
        nt = L % Bk
        for name in tails:
            row = (b * H + h) * Bk * D * 2
            gpu = tails[name][row:row + nt * D * 2]
            ora = np.ascontiguousarray(getattr(hc, name)).view(np.uint8).reshape(-1)[:nt * D * 2]
            assert np.array_equal(gpu, ora), (name, b, h)


@pytest.mark.parametrize("case", sorted(CASES))
def test_paged_matches_oracle_and_dense(case):
    import torch
    import oracle
    import quantized_decode_attn_amd as kvq
    cfg, steps = CASES[case]
    B, H, Hq, D = cfg["batch"], cfg["kv_heads"], cfg["q_heads"], cfg["head_dim"]
    steps = np.array(steps)
    final = steps.sum(axis=0)
    rng = np.random.default_rng(7)
    k, v = synth.gen_tensor(cfg, synth.TENSOR_K), synth.gen_tensor(cfg, synth.TENSOR_V)
    lut = _lut(cfg)
    lut_t = None if lut is None else upload(lut)
    table, P = _table(cfg, final, rng)
    dev = torch.device("cuda:0")
    paged = kvq.PagedCache(cfg, num_blocks=P, block_table=torch.from_numpy(table).to(dev), device=dev, lut=lut_t)
    dense = kvq.PagedCache(cfg, device=dev, lut=lut_t)      # per-sequence lengths, dense slots
    ko = oracle.kout(cfg)
    say("case", case, "lengths", list(final), "pool", P)
    done = np.zeros(B, np.int64)
    for si, cnt in enumerate(steps):
        n_max = int(cnt.max())
        if n_max:
            kn = np.zeros((B, H, n_max, D), np.uint16)
            vn = np.zeros((B, H, n_max, D), np.uint16)
            for b in range(B):
                kn[b, :, :cnt[b]] = k[b, :, done[b]:done[b] + cnt[b]]
                vn[b, :, :cnt[b]] = v[b, :, done[b]:done[b] + cnt[b]]
            kd, vd = upload(kn), upload(vn)
            paged.append_seqs(kd, vd, cnt)
            dense.append_seqs(kd, vd, cnt)
        done += cnt
        assert paged.lengths == list(done) == dense.lengths
        if si >= 1 and (done > 0).all():
            q = synth.gen_q(cfg, seed=si)
            qd = upload(q)
            a = paged.decode(qd).cpu().numpy()
            d = dense.decode(qd).cpu().numpy()
            ref, heads = _oracle_decode(cfg, k, v, lut, list(done), q)
            err = float(np.abs(a.astype(np.float64) - ref).max())
            say("  step", si, "lengths", list(done), "max abs err", err)
            assert err <= TOL
            assert np.array_equal(a.view(np.uint32), d.view(np.uint32))
    torch.cuda.synchronize()
    _compare_blocks(paged, table, cfg, ko, heads, list(done))
    _compare_blocks(dense, None, cfg, ko, heads, list(done))


@pytest.mark.parametrize("case", ["mha_v4", "gqa_csr", "generic_gqa_d64"])
def test_equal_lengths_match_the_dense_cache(case):
    """All sequences at one length: the paged cache's decode equals the plain dense
    cache's within 2e-5, the bound of a change of split grouping (the per-sequence
    kernels give a sequence ceil(blocks / ceil((T / Bk) / S)) splits)."""
    import torch
    import quantized_decode_attn_amd as kvq
    from _gpu_util import build_gpu_cache
    cfg = dict(CASES[case][0])
    B, H = cfg["batch"], cfg["kv_heads"]
    T = cfg["capacity"] - cfg["k_block"] // 2 - 3
    k, v = synth.gen_tensor(cfg, synth.TENSOR_K), synth.gen_tensor(cfg, synth.TENSOR_V)
    lut = _lut(cfg)
    lut_t = None if lut is None else upload(lut)
    rng = np.random.default_rng(3)
    table, P = _table(cfg, [T] * B, rng)
    dev = torch.device("cuda:0")
    paged = kvq.PagedCache(cfg, num_blocks=P, block_table=torch.from_numpy(table).to(dev), device=dev, lut=lut_t)
    for t0, t1 in ((0, 200), (200, 201), (201, T)):
        paged.append_seqs(upload(k[:, :, t0:t1]), upload(v[:, :, t0:t1]), [t1 - t0] * B)
    plain = build_gpu_cache(cfg, k[:, :, :T], v[:, :, :T], [200, 1, T - 201], lut)
    q = upload(synth.gen_q(cfg, seed=5))
    for S in (0, 3):
        a = paged.decode(q, num_splits=S).cpu().numpy()
        b = plain.decode(q, q_pos=T - 1, num_splits=S).cpu().numpy()
        say("case", case, "splits", S, "max abs diff", float(np.abs(a - b).max()))
        assert float(np.abs(a - b).max()) <= 2e-5


def test_paged_calls_and_checks():
    """What a per-sequence cache refuses, and that a refused call changes nothing."""
    import torch
    import quantized_decode_attn_amd as kvq
    cfg = dict(CASES["mha_v4"][0])
    B, H, D = cfg["batch"], cfg["kv_heads"], cfg["head_dim"]
    dev = torch.device("cuda:0")
    table, P = _table(cfg, [cfg["capacity"]] * B, np.random.default_rng(1))
    paged = kvq.PagedCache(cfg, num_blocks=P, block_table=torch.from_numpy(table).to(dev), device=dev)
    k = upload(synth.gen_tensor(cfg, synth.TENSOR_K, 0, 8))
    paged.append_seqs(k, k, [8, 0, 3])
    assert paged.lengths == [8, 0, 3]
    q = upload(synth.gen_q(cfg))
    with pytest.raises(kvq.KvqError):                # a sequence without tokens
        paged.decode(q)
    import ctypes
    counts = torch.tensor([8, 0, 0], dtype=torch.int64, device=dev)
    with pytest.raises(kvq.KvqError):                # a sequence past the capacity
        kvq.kvq_quantize_append_seqs(paged.desc, k, k, 8, (ctypes.c_int64 * B)(8, 0, cfg["capacity"]), counts)
    with pytest.raises(kvq.KvqError):                # a count above the input's rows
        kvq.kvq_quantize_append_seqs(paged.desc, k, k, 8, (ctypes.c_int64 * B)(9, 0, 0), counts)
    assert paged.lengths == [8, 0, 3]
    for bad in (lambda: kvq.kvq_chunk_attention(paged.desc, q, 1, 0, q, q, 1 << 20, 0),
                lambda: kvq.kvq_dequantize(paged.desc, 0, 0, 1, q)):
        with pytest.raises(kvq.KvqError):
            bad()
    torch.cuda.synchronize()
