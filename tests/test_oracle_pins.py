"""Pins of the CPU oracle against what the pages and plain mathematics fix.

Nothing here compares the oracle with a retyped copy of itself: every check is a
page figure (tests/golden/page_figures.json), a library routine (numpy's fp16
cast and quantile), a brute-force search over all codes, a closed form, or an
invariant of the definition.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "page_figures.json")))


def tiny(**kw):
    c = dict(batch=1, q_heads=1, kv_heads=1, head_dim=8, tokens=16, k_bits=4, k_mode=0,
             k_block=8, v_bits=4, v_group=8, clip_quantile=0.0, outlier_pct=0, rope_theta=10000.0)
    c.update(kw)
    c.setdefault("capacity", c["tokens"])
    return c


def f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def hval(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------- fp16
def test_h2f_exhaustive(orc):
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.h2f(allh)
    ref = allh.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f2h_rn_matches_numpy_cast(orc):
    rng = np.random.default_rng(7)
    e = rng.integers(-30, 17, 200000)
    x = (rng.random(200000) + 0.5) * np.exp2(e) * rng.choice([-1, 1], 200000)
    x = x.astype(np.float32)
    # exact midpoints between neighbouring fp16 values (ties) and boundary values
    h = rng.integers(0, 0x7bff, 50000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float32)
    hi = (h + 1).view(np.float16).astype(np.float32)
    mids = ((lo.astype(np.float64) + hi.astype(np.float64)) / 2).astype(np.float32)
    special = np.array([0.0, -0.0, 65504, 65519.99, 65520, 1e9, -1e9, 2 ** -24, 2 ** -25,
                        3 * 2 ** -26, 2 ** -14, 6.1e-5, np.inf, -np.inf], np.float32)
    x = np.concatenate([x, mids, -mids, special])
    got = orc.f2h(x, "rn")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f2h_directed_rounding(orc):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-26, 14, 100000))).astype(np.float32)
    x = np.concatenate([x, f16([0.5, -3.25, 1024.0]).view(np.float16).astype(np.float32),
                        np.array([0.0, 1e-9, -1e-9], np.float32)])
    rd = hval(orc.f2h(x, "rd"))
    ru = hval(orc.f2h(x, "ru"))
    rn = hval(orc.f2h(x, "rn"))
    xd = x.astype(np.float64)
    assert np.all(rd <= xd) and np.all(ru >= xd)
    exact = rd == xd
    assert np.all(ru[exact] == xd[exact])
    # otherwise rd and ru are neighbours in fp16
    ne = ~exact
    nxt = np.nextafter(rd[ne].astype(np.float16), np.float16(np.inf)).astype(np.float64)
    assert np.all(nxt == ru[ne])
    assert np.all((rn == rd) | (rn == ru))


# --------------------------------------------------------------------------- sizes
def test_kv_size_worked_example(orc):
    for key in ("kv_size_example", "kv_size_example_batch4"):
        g = GOLD[key]
        v = orc.kv_bytes(g["layers"], g["batch"], g["tokens"], g["hidden"], g["bits"])
        assert v == 2 * g["layers"] * g["batch"] * g["tokens"] * g["hidden"] * 2
        assert abs(v - g["page_value_bytes_approx"]) / g["page_value_bytes_approx"] < 0.08
    assert orc.kv_bytes(32, 1, 2048, 4096, 16) == 2 ** 30


def test_int4_is_quarter_of_fp16(orc):
    g = GOLD["fp16_to_int4_factor"]
    for kb, frac in ((4, 1 / g["factor"]), (3, 3 / 16), (2, 1 / 8)):
        c = tiny(head_dim=128, k_block=128, tokens=1024, k_bits=kb, v_group=128)
        lay = orc.layout(c)
        fp16 = c["tokens"] * c["head_dim"] * 2
        assert lay["k_codes"] / fp16 == frac
    c = tiny(head_dim=128, k_block=128, tokens=1024, v_group=128)
    assert orc.layout(c)["v_codes"] / (1024 * 128 * 2) == 0.25


def test_int4_has_16_states(orc):
    g = GOLD["int4_states"]
    c = tiny(head_dim=8, k_block=32, tokens=32)
    x = np.linspace(-3, 5, 32 * 8).reshape(32, 8)
    hc = orc.HeadCache(c).build(f16(x), f16(x))
    codes = _codes_uniform_k(hc, c)
    assert sorted(set(codes.ravel().tolist())) == list(range(g["states"]))


def test_memory_fraction_near_quarter(orc):
    g = GOLD["int4_memory_target"]
    import synth
    c = synth.config("c1")
    lay = orc.layout(c)
    tail = lay["k_tail"] + lay["v_tail"]
    frac = (sum(lay.values()) - tail) / (2 * c["batch"] * c["kv_heads"] * c["tokens"] * c["head_dim"] * 2)
    assert abs(frac - g["fraction_of_fp16"]) < 0.02        # 26.6 % with fp16 scales and zeros
    per_token_head = (sum(lay.values()) - tail) / (c["batch"] * c["kv_heads"] * c["tokens"])
    assert per_token_head == 136                            # 64 + 64 code bytes, 4 + 4 metadata bytes


# --------------------------------------------------------------------------- helpers
def _deq(hc, which):
    return hc.dequantize(which).astype(np.float64)


def _codes_uniform_k(hc, c):
    """Recover K codes from the dequantized values (fmaf(c, s, z) with s > 0)."""
    D, Bk = c["head_dim"], c["k_block"]
    n = hc.length // Bk * Bk
    x = _deq(hc, 0)[:n]
    s = np.repeat(hval(hc.k_scale), Bk, axis=0)[:n]
    z = np.repeat(hval(hc.k_zero), Bk, axis=0)[:n]
    with np.errstate(invalid="ignore", divide="ignore"):
        cc = np.where(s > 0, np.rint((x - z) / np.where(s > 0, s, 1)), 0)
    return cc.astype(np.int64)


def _rand_block(rng, T, D, scale=1.0, heavy=False):
    std = np.exp(rng.normal(0, 0.5, D)) * scale
    x = rng.standard_normal((T, D)) * std
    if heavy:
        m = rng.random((T, D)) < 0.02
        x[m] = np.clip(10 * rng.standard_t(3, m.sum()), -200, 200)
    return f16(x)


def _outlier_mask(hc, c, which):
    T = hc.length // c["k_block"] * c["k_block"]
    m = np.zeros((T, c["head_dim"]), bool)
    if hc.kout:
        col = (hc.v_col if which else hc.k_col)[:T * hc.kout].reshape(T, hc.kout)
        m[np.arange(T)[:, None], col] = True
    return m


# --------------------------------------------------------------------------- uniform quantizer
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("pct", [0, 5])
def test_uniform_codes_are_nearest_grid_points(orc, bits, pct):
    """Brute force over every code: the chosen code minimises |x - (c*s + z)| (exact
    ties excluded), for K per channel and V per token group."""
    rng = np.random.default_rng(bits * 10 + pct)
    vb = 4 if bits == 3 else bits
    c = tiny(head_dim=32, k_block=16, tokens=64, k_bits=bits, v_bits=vb, v_group=16, outlier_pct=pct)
    k = _rand_block(rng, 64, 32, heavy=pct > 0)
    v = _rand_block(rng, 64, 32, heavy=pct > 0)
    hc = orc.HeadCache(c).build(k, v)
    for which, src, L in ((0, k, (1 << bits) - 1), (1, v, (1 << vb) - 1)):
        x = hval(src)
        xh = _deq(hc, which)
        if which == 0:
            s = np.repeat(hval(hc.k_scale), 16, axis=0)
            z = np.repeat(hval(hc.k_zero), 16, axis=0)
        else:
            s = np.repeat(hval(hc.v_scale), 16, axis=1)
            z = np.repeat(hval(hc.v_zero), 16, axis=1)
        dense = ~_outlier_mask(hc, c, which) & (s > 0)
        grid = z[..., None] + np.arange(L + 1) * s[..., None]              # fp64 grid
        best = np.argmin(np.abs(x[..., None] - grid), axis=-1)
        chosen = np.rint((xh - z) / np.where(s > 0, s, 1))
        u = (x - z) / np.where(s > 0, s, 1)
        tie = np.abs(u - np.floor(u) - 0.5) < 1e-5
        ok = dense & ~tie
        assert ok.sum() > 0.9 * dense.sum()
        assert np.array_equal(best[ok], chosen[ok])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_uniform_error_bound_half_scale(orc, bits):
    """|x - dequant(x)| <= s/2 (+ fp32 evaluation slack) for unclipped dense values."""
    rng = np.random.default_rng(100 + bits)
    vb = 4 if bits == 3 else bits
    c = tiny(head_dim=64, k_block=32, tokens=96, k_bits=bits, v_bits=vb, v_group=32, outlier_pct=2)
    k = _rand_block(rng, 96, 64, heavy=True)
    v = _rand_block(rng, 96, 64, heavy=True)
    hc = orc.HeadCache(c).build(k, v)
    for which, src in ((0, k), (1, v)):
        x = hval(src)
        xh = _deq(hc, which)
        if which == 0:
            s = np.repeat(hval(hc.k_scale), 32, axis=0)
            z = np.repeat(hval(hc.k_zero), 32, axis=0)
        else:
            s = np.repeat(hval(hc.v_scale), 32, axis=1)
            z = np.repeat(hval(hc.v_zero), 32, axis=1)
        m = _outlier_mask(hc, c, which)
        ulp = np.spacing(np.maximum(np.abs(x), np.abs(z)).astype(np.float32)).astype(np.float64)
        err = np.abs(x - xh)
        assert np.all(err[~m] <= s[~m] / 2 + 4 * ulp[~m])
        assert np.array_equal(xh[m], x[m])                         # outliers are exact


def test_metadata_invariants(orc):
    """zero = largest fp16 <= group min, scale = smallest fp16 >= (max - zero)/L;
    the group min codes to 0 and the group max to L; outliers take no part."""
    rng = np.random.default_rng(5)
    c = tiny(head_dim=64, k_block=32, tokens=64, v_group=16, outlier_pct=3)
    k = _rand_block(rng, 64, 64, heavy=True)
    v = _rand_block(rng, 64, 64, heavy=True)
    hc = orc.HeadCache(c).build(k, v)
    L = 15
    mk = _outlier_mask(hc, c, 0)
    mv = _outlier_mask(hc, c, 1)
    x = hval(k)
    codes = _codes_uniform_k(hc, c)
    for n in range(2):
        for ch in range(64):
            sel = ~mk[n * 32:(n + 1) * 32, ch]
            vals = x[n * 32:(n + 1) * 32, ch][sel]
            z = hval(hc.k_zero[n, ch])
            s = hval(hc.k_scale[n, ch])
            lo, hi = vals.min(), vals.max()
            assert z <= lo < np.nextafter(np.float16(z), np.float16(np.inf)).astype(np.float64)
            r = np.float32(np.float32(hi - z) / np.float32(L))
            assert s >= r and np.nextafter(np.float16(s), np.float16(-np.inf)) < r
            cc = codes[n * 32:(n + 1) * 32, ch][sel]
            assert cc[np.argmin(vals)] == 0 and cc[np.argmax(vals)] == L
    xv = hval(v)
    for t in range(64):
        for g in range(4):
            sel = ~mv[t, g * 16:(g + 1) * 16]
            vals = xv[t, g * 16:(g + 1) * 16][sel]
            z = hval(hc.v_zero[t, g])
            assert z <= vals.min() < np.nextafter(np.float16(z), np.float16(np.inf)).astype(np.float64)


def test_metadata_invariants_after_clipping(orc):
    """With clipping the group minimum is the fp32 threshold -t, not an fp16 value:
    the zero-point must still be the largest fp16 not above it."""
    rng = np.random.default_rng(6)
    c = tiny(head_dim=64, k_block=32, tokens=64, v_group=64, clip_quantile=0.97)
    k = _rand_block(rng, 64, 64, heavy=True)
    hc = orc.HeadCache(c).build(k, k)
    hits = 0
    for n in range(2):
        blk = k[n * 32:(n + 1) * 32]
        t = np.float32(orc.clip_threshold(blk, np.float32(0.97)))
        d = np.clip(hval(blk).astype(np.float32), -t, t).astype(np.float64)
        for ch in range(64):
            lo = d[:, ch].min()
            z = hval(hc.k_zero[n, ch])
            assert z <= lo < np.nextafter(np.float16(z), np.float16(np.inf)).astype(np.float64)
            hits += lo == -t
        for t_ in range(32):
            lo = d[t_].min()
            z = hval(hc.v_zero[n * 32 + t_, 0])
            assert z <= lo < np.nextafter(np.float16(z), np.float16(np.inf)).astype(np.float64)
    assert hits > 0


def test_exact_ties_round_half_to_even(orc):
    """Group with zero 0 and scale 1 (values 0 and 15 present); x = k + 1/2 must take
    the even neighbour."""
    c = tiny(head_dim=32, k_block=8, tokens=8, v_group=32)
    v = np.zeros((8, 32))
    v[:, 0], v[:, 1] = 0.0, 15.0
    v[:, 2:17] = np.arange(15) + 0.5
    hc = orc.HeadCache(c).build(f16(v), f16(v))
    got = _deq(hc, 1)[:, 2:17]
    want = np.array([k if k % 2 == 0 else k + 1 for k in range(15)], np.float64)
    assert np.all(hval(hc.v_scale) == 1.0) and np.all(hval(hc.v_zero) == 0.0)
    assert np.array_equal(got, np.tile(want, (8, 1)))


def test_constant_and_empty_groups(orc):
    c = tiny(head_dim=8, k_block=8, tokens=8, v_group=4, outlier_pct=13)   # k_out = 2
    k = np.full((8, 8), 1.25)
    k[:, 3] = 500.0 + np.arange(8)             # channel 3 is the largest of every token
    k[:, 6] = 400.0                            # channel 6 is the second largest
    v = np.full((8, 8), -0.75)
    v[:, 0] = 9.0
    v[:, 1] = 8.0                              # group 0 keeps channels 2, 3 only
    hc = orc.HeadCache(c).build(f16(k), f16(v))
    assert hc.k_scale[0, 3] == 0 and hc.k_zero[0, 3] == 0          # empty channel
    assert hc.k_scale[0, 0] == 0 and hval(hc.k_zero[0, 0]) == 1.25  # constant channel
    assert np.all(hc.v_scale == 0) and np.all(hval(hc.v_zero) == -0.75)
    assert np.array_equal(_deq(hc, 0), hval(f16(k)))
    assert np.array_equal(_deq(hc, 1), hval(f16(v)))


# --------------------------------------------------------------------------- outliers
def test_outliers_are_top_k_by_magnitude(orc):
    rng = np.random.default_rng(11)
    c = tiny(head_dim=128, k_block=16, tokens=64, v_group=128, outlier_pct=1)
    assert orc.kout(c) == 2 and orc.kout(tiny(head_dim=64, outlier_pct=1)) == 1
    k = _rand_block(rng, 64, 128, heavy=True)
    v = _rand_block(rng, 64, 128, heavy=True)
    k[5, [10, 90]] = f16([7.0, -7.0])           # exact magnitude tie: both must be taken
    k[5, 20] = f16(1e3)
    hc = orc.HeadCache(c).build(k, v)
    for which, src in ((0, k), (1, v)):
        col = (hc.v_col if which else hc.k_col).reshape(64, 2)
        val = (hc.v_val if which else hc.k_val).reshape(64, 2)
        rp = hc.v_rowptr if which else hc.k_rowptr
        assert rp[0] == 0 and np.all(np.diff(rp) == 2)
        mag = (src & 0x7FFF).astype(np.int64)
        for t in range(64):
            order = np.lexsort((np.arange(128), -mag[t]))   # |x| descending, then column ascending
            want = np.sort(order[:2])
            assert np.array_equal(col[t], want)
            assert np.all(np.diff(col[t].astype(int)) > 0)
            assert np.array_equal(val[t], src[t, want])
    assert set(hc.k_col.reshape(64, 2)[5]) == {20, 10}


# --------------------------------------------------------------------------- clip
@pytest.mark.parametrize("q", [0.99, 0.5, 0.9])
def test_clip_threshold_equals_numpy_quantile(orc, q):
    rng = np.random.default_rng(int(q * 100))
    for trial in range(20):
        n = int(rng.integers(2, 5000))
        x = rng.standard_normal(n) * np.exp(rng.normal(0, 2))
        if trial % 3 == 0:
            x = np.round(x * 4) / 4                              # many exact duplicates
        b = f16(x)
        t = orc.clip_threshold(b, np.float32(q))
        ref = np.quantile(np.abs(hval(b)), np.float64(np.float32(q)), method="linear")
        assert abs(t - ref) <= np.spacing(np.float32(ref))


def test_clip_bounds_dense_values(orc):
    rng = np.random.default_rng(3)
    c = tiny(head_dim=64, k_block=32, tokens=64, v_group=64, clip_quantile=0.99, outlier_pct=1)
    k = _rand_block(rng, 64, 64, heavy=True)
    v = _rand_block(rng, 64, 64, heavy=True)
    hc = orc.HeadCache(c).build(k, v)
    for which, src in ((0, k), (1, v)):
        xh = _deq(hc, which)
        m = _outlier_mask(hc, c, which)
        for n in range(2):
            blk = src[n * 32:(n + 1) * 32]
            t = np.quantile(np.abs(hval(blk)), np.float64(np.float32(0.99)), method="linear")
            s = hval(hc.k_scale[n]).max() if which == 0 else hval(hc.v_scale[n * 32:(n + 1) * 32]).max()
            dense = xh[n * 32:(n + 1) * 32][~m[n * 32:(n + 1) * 32]]
            assert np.abs(dense).max() <= t + s / 2 + 1e-3
            assert np.abs(hval(blk)).max() > t                     # something was clipped


# --------------------------------------------------------------------------- non-uniform codebook
def _lut_cfg(D=16, kb=3, Bk=16, T=32):
    return tiny(head_dim=D, k_block=Bk, tokens=T, k_bits=kb, k_mode=1, v_bits=4, v_group=D)


def test_codebook_codes_are_nearest_centroid(orc):
    rng = np.random.default_rng(21)
    c = _lut_cfg()
    lut = np.sort(rng.standard_normal((16, 8)) * 1.5, axis=1).astype(np.float16).view(np.uint16)
    k = _rand_block(rng, 32, 16)
    v = _rand_block(rng, 32, 16)
    hc = orc.HeadCache(c, lut).build(k, v)
    x = hval(k)
    xh = _deq(hc, 0)
    C = hval(lut)                                               # [D][8]
    best = np.argmin(np.abs(x[:, :, None] - C[None]), axis=2)
    got = np.argmax(xh[:, :, None] == C[None], axis=2)
    mids = (C[:, :-1] + C[:, 1:]) / 2
    near = np.min(np.abs(x[:, :, None] - mids[None]), axis=2) < 1e-6 * (1 + np.abs(x))
    assert np.array_equal(best[~near], got[~near])
    assert np.all(np.isin(xh, C))


def test_evenly_spaced_codebook_is_uniform_rounding(orc):
    rng = np.random.default_rng(22)
    c = _lut_cfg(kb=4)
    z, s = -2.0, 0.25
    lut = np.tile(f16(z + s * np.arange(16)), (16, 1))
    k = _rand_block(rng, 32, 16)
    k[3] = f16(z + s * (np.arange(16) % 15 + 0.5))             # exact midpoints: lower code wins
    hc = orc.HeadCache(c, lut).build(k, k)
    u = (hval(k) - z) / s
    want = np.clip(np.floor(u + 0.5 - 1e-12), 0, 15)           # nearest, ties to lower
    got = (_deq(hc, 0) - z) / s
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------- packing
def _identity_lut(D, kb):
    return np.tile(f16(np.arange(1 << kb)), (D, 1))


@pytest.mark.parametrize("kb,row,want", [
    (4, [1, 2, 3, 4], [0x31, 0x42]),            # bytes hold channel pairs (0, 2) and (1, 3)
    (3, [1, 2, 3, 4, 5, 6, 7, 0], [0xA9, 0xBC, 0x13]),   # 3-bit codes straddle bytes, LSB first
    (2, [1, 2, 3, 0], [0x2D]),
])
def test_key_row_known_bytes(orc, kb, row, want):
    D = len(row)
    c = tiny(head_dim=D, k_block=8, tokens=8, k_bits=kb, k_mode=1, v_group=D)
    k = np.tile(np.asarray(row, np.float64), (8, 1))
    hc = orc.HeadCache(c, _identity_lut(D, kb)).build(f16(k), f16(k))
    rb = D * kb // 8
    assert list(hc.k_codes[:rb]) == want
    assert np.array_equal(hc.k_codes.reshape(8, rb), np.tile(np.asarray(want, np.uint8), (8, 1)))


def test_value_words_known_bytes(orc):
    c = tiny(head_dim=2, k_block=8, tokens=8, v_group=2)
    v = np.array([[0, 15], [15, 0]] * 4, np.float64)             # per-token codes equal the values
    hc = orc.HeadCache(c).build(f16(v), f16(v))
    assert list(hc.v_codes) == [0xF0] * 4 + [0x0F] * 4          # word(ch0), word(ch1); token t at bits 4t
    c2 = tiny(head_dim=2, k_block=16, tokens=16, v_bits=2, v_group=2)
    v2 = np.array([[0, 3], [3, 0]] * 8, np.float64)
    hc2 = orc.HeadCache(c2).build(f16(v2), f16(v2))
    assert list(hc2.v_codes) == [0xCC] * 4 + [0x33] * 4


@pytest.mark.parametrize("kb", [2, 3, 4])
def test_key_pack_roundtrip(orc, kb):
    rng = np.random.default_rng(kb)
    c = tiny(head_dim=64, k_block=16, tokens=48, k_bits=kb, k_mode=1, v_group=64)
    codes = rng.integers(0, 1 << kb, (48, 64))
    hc = orc.HeadCache(c, _identity_lut(64, kb)).build(f16(codes), f16(codes))
    assert np.array_equal(_deq(hc, 0), codes.astype(np.float64))


# --------------------------------------------------------------------------- attention
def _softmax_attn(qr, kr, v, D):
    s = kr @ qr / math.sqrt(D)
    w = np.exp(s - s.max())
    return (w[:, None] * v).sum(0) / w.sum()


def _rot_matrix(pos, D, theta):
    """Full D x D rotary matrix built from 2x2 rotations on channel pairs (i, i + D/2)."""
    R = np.zeros((D, D))
    h = D // 2
    for i in range(h):
        a = pos * theta ** (-2.0 * i / D)
        R[i, i], R[i, i + h], R[i + h, i], R[i + h, i + h] = np.cos(a), -np.sin(a), np.sin(a), np.cos(a)
    return R


def test_rope_pairing_and_direction_closed_form(orc):
    """D = 4, tail-only cache (exact values): key e_2 at position 1 against query e_0
    at position 0 scores -sin(1)/2; key e_3 against e_1 scores -sin(0.01)/2."""
    c = tiny(head_dim=4, k_block=8, tokens=2, v_group=4)
    for qch, kch, ang in ((0, 2, 1.0), (1, 3, 0.01)):
        k = np.zeros((2, 4)); k[0, qch] = 1.0; k[1, kch] = 1.0
        v = np.zeros((2, 4)); v[0, 0] = 1.0; v[1, 1] = 1.0
        hc = orc.HeadCache(c).build(f16(k), f16(v))
        q = np.zeros(4); q[qch] = 1.0
        out = hc.decode(f16(q), q_pos=0)
        s0, s1 = 0.5, -math.sin(ang) / 2
        w0, w1 = math.exp(s0), math.exp(s1)
        assert abs(out[0] - w0 / (w0 + w1)) < 1e-12 and abs(out[1] - w1 / (w0 + w1)) < 1e-12


def test_attention_closed_forms(orc):
    rng = np.random.default_rng(31)
    c = tiny(head_dim=32, k_block=16, tokens=72, v_group=16, outlier_pct=4)
    k = _rand_block(rng, 72, 32, heavy=True)
    v = _rand_block(rng, 72, 32, heavy=True)
    hc = orc.HeadCache(c).build(k, v)
    vh = _deq(hc, 1)
    out = hc.decode(f16(np.zeros(32)), q_pos=71)                # q = 0: uniform weights
    assert np.allclose(out, vh.mean(0), rtol=0, atol=1e-12)
    h1 = orc.HeadCache(tiny(head_dim=32, k_block=16, tokens=1, v_group=16)).build(k[:1], v[:1])
    assert np.array_equal(h1.decode(f16(rng.standard_normal(32))), hval(v[0]))   # one token
    vc = np.full((72, 32), 0.8125)
    hcc = orc.HeadCache(c).build(k, f16(vc))
    assert np.allclose(hcc.decode(f16(rng.standard_normal(32))), 0.8125, rtol=0, atol=1e-12)


def _on_grid(rng, T, D, Bk, L, per_channel):
    """Values that the uniform quantizer must reproduce exactly: each group holds
    zero + c * scale with zero a multiple of 1/64, a power-of-two scale and both end
    codes present, so every value is exact in fp16."""
    x = np.empty((T, D))
    for n in range(T // Bk):
        if per_channel:
            for ch in range(D):
                z = float(rng.integers(-192, 1)) / 64
                s = 2.0 ** rng.integers(-5, -1)
                cc = rng.integers(0, L + 1, Bk); cc[0], cc[1] = 0, L
                x[n * Bk:(n + 1) * Bk, ch] = z + cc * s
        else:
            for t in range(n * Bk, (n + 1) * Bk):
                z = float(rng.integers(-192, 1)) / 64
                s = 2.0 ** rng.integers(-5, -1)
                cc = rng.integers(0, L + 1, D); cc[0], cc[1] = 0, L
                x[t] = z + cc * s
    return x


@pytest.mark.parametrize("bits", [2, 4])
def test_quantized_attention_equals_textbook_on_grid(orc, bits):
    """On-grid caches dequantize exactly, so the oracle must equal plain fp64
    softmax attention with rotary matrices applied to the raw inputs."""
    rng = np.random.default_rng(40 + bits)
    D, Bk, T = 16, 16, 48
    L = (1 << bits) - 1
    c = tiny(head_dim=D, k_block=Bk, tokens=T + 5, k_bits=bits, v_bits=bits, v_group=D, capacity=64)
    k = np.concatenate([_on_grid(rng, T, D, Bk, L, True), rng.standard_normal((5, D))])
    v = np.concatenate([_on_grid(rng, T, D, Bk, L, False), rng.standard_normal((5, D))])
    kb, vb = f16(k), f16(v)
    hc = orc.HeadCache(c).build(kb, vb)
    assert np.array_equal(_deq(hc, 0), hval(kb)) and np.array_equal(_deq(hc, 1), hval(vb))
    q = f16(rng.standard_normal(D) * 2)
    for qp in (T + 4, 200, 3):
        out = hc.decode(q, q_pos=qp)
        qr = _rot_matrix(qp, D, 10000.0) @ hval(q)
        kr = np.stack([_rot_matrix(t, D, 10000.0) @ hval(kb[t]) for t in range(T + 5)])
        ref = _softmax_attn(qr, kr, hval(vb), D)
        assert np.max(np.abs(out - ref)) < 1e-12


def test_blocks_are_independent_of_later_tokens(orc):
    rng = np.random.default_rng(50)
    c = tiny(head_dim=16, k_block=16, tokens=64, v_group=8, outlier_pct=7, clip_quantile=0.9)
    k = _rand_block(rng, 64, 16, heavy=True)
    v = _rand_block(rng, 64, 16, heavy=True)
    a = orc.HeadCache(c).build(k[:37], v[:37])
    b = orc.HeadCache(c).build(k, v)
    n = 32
    assert np.array_equal(a.k_codes[:n * 8], b.k_codes[:n * 8])
    assert np.array_equal(a.v_codes[:n * 8], b.v_codes[:n * 8])
    assert np.array_equal(a.k_scale[:2], b.k_scale[:2]) and np.array_equal(a.v_zero[:n], b.v_zero[:n])
    assert np.array_equal(a.k_tail[:5], k[32:37]) and np.array_equal(a.v_tail[:5], v[32:37])
    assert np.array_equal(a.dequantize(0, 0, 32), b.dequantize(0, 0, 32))
    assert np.array_equal(a.dequantize(0, 32, 37), hval(k[32:37]).astype(np.float32))


# --------------------------------------------------------------------------- chunk of queries
def test_chunk_equals_textbook_causal_attention_on_grid(orc):
    """Query j of a chunk sits at position q_pos + j and sees the tokens t <= q_pos + j.
    On an on-grid cache (exact dequantization) every row must equal plain fp64 softmax
    attention over that prefix, with rotary matrices applied to the raw inputs; rows
    at or past the last token see the whole cache."""
    rng = np.random.default_rng(61)
    D, Bk, T = 16, 16, 48
    c = tiny(head_dim=D, k_block=Bk, tokens=T + 5, v_group=D, capacity=64)
    k = np.concatenate([_on_grid(rng, T, D, Bk, 15, True), rng.standard_normal((5, D))])
    v = np.concatenate([_on_grid(rng, T, D, Bk, 15, False), rng.standard_normal((5, D))])
    kb, vb = f16(k), f16(v)
    hc = orc.HeadCache(c).build(kb, vb)
    kr_all = [hval(kb[t]) for t in range(T + 5)]
    for q_pos, nq in ((14, 5), (44, 12), (0, 3)):
        q = f16(rng.standard_normal((nq, D)) * 2)
        out = hc.chunk(q, q_pos)
        assert out.shape == (nq, D)
        for j in range(nq):
            p = q_pos + j
            n = min(p + 1, T + 5)
            qr = _rot_matrix(p, D, 10000.0) @ hval(q[j])
            kr = np.stack([_rot_matrix(t, D, 10000.0) @ kr_all[t] for t in range(n)])
            ref = _softmax_attn(qr, kr, hval(vb[:n]), D)
            assert np.max(np.abs(out[j] - ref)) < 1e-12, (q_pos, j)


def test_chunk_zero_queries_average_their_prefix(orc):
    """q = 0 gives equal weights, so row j is the mean of the first min(q_pos + j + 1, T)
    dequantized values: the causal boundary is visible in the output."""
    rng = np.random.default_rng(62)
    c = tiny(head_dim=32, k_block=16, tokens=72, v_group=16, outlier_pct=4, clip_quantile=0.9)
    k = _rand_block(rng, 72, 32, heavy=True)
    v = _rand_block(rng, 72, 32, heavy=True)
    hc = orc.HeadCache(c).build(k, v)
    vh = _deq(hc, 1)
    out = hc.chunk(f16(np.zeros((9, 32))), 62)
    for j in range(9):
        n = min(63 + j, 72)
        assert np.allclose(out[j], vh[:n].mean(0), rtol=0, atol=1e-12), j


def test_chunk_rows_equal_decode_over_the_prefix_cache(orc):
    """Blocks are quantized independently of later tokens, so a cache built from the
    first n tokens holds the same dequantized values whenever n is a block boundary or
    lies past the last one (then the difference is only the shorter fp16 tail).  Row j
    of a chunk must equal single-query decode over such a prefix cache; with nq = 1 at
    the last position it is the decode over the whole cache."""
    rng = np.random.default_rng(63)
    c = tiny(head_dim=16, k_block=16, tokens=75, v_group=8, outlier_pct=7, clip_quantile=0.9)
    k = _rand_block(rng, 75, 16, heavy=True)
    v = _rand_block(rng, 75, 16, heavy=True)
    full = orc.HeadCache(c).build(k, v)
    q = f16(rng.standard_normal((12, 16)))
    q_pos = 63                                             # rows see 64 (a boundary) .. 75 tokens
    out = full.chunk(q, q_pos)
    for j in range(12):
        n = min(q_pos + j + 1, 75)
        pre = orc.HeadCache(c).build(k[:n], v[:n])
        ref = pre.decode(q[j], q_pos=q_pos + j)
        assert np.max(np.abs(out[j] - ref)) < 1e-12, j
    last = full.chunk(q[:1], 74)
    assert np.array_equal(last[0], full.decode(q[0], q_pos=74))


def test_chunk_ignores_tokens_after_each_query(orc):
    """Changing the newest (fp16 tail) tokens leaves every row that does not see them
    unchanged and changes the rows that do."""
    rng = np.random.default_rng(64)
    c = tiny(head_dim=16, k_block=16, tokens=45, v_group=16)
    k = _rand_block(rng, 45, 16)
    v = _rand_block(rng, 45, 16)
    k2, v2 = k.copy(), v.copy()
    k2[40:] = f16(rng.standard_normal((5, 16)) * 3)
    v2[40:] = f16(rng.standard_normal((5, 16)) * 3)
    a = orc.HeadCache(c).build(k, v)
    b = orc.HeadCache(c).build(k2, v2)
    q = f16(rng.standard_normal((8, 16)))
    oa, ob = a.chunk(q, 35), b.chunk(q, 35)               # rows see 36 .. 43 tokens
    assert np.array_equal(oa[:5], ob[:5])                  # rows 0..4 see t <= 39
    assert all(np.max(np.abs(oa[j] - ob[j])) > 1e-6 for j in range(5, 8))


# --------------------------------------------------------------------------- keys kept in fp16
# [TQ] section 3.2: the few key vectors judged important by their own norm keep fp16, the
# rest are quantized; section 6.1: the L2 norm directly.
def _exact_norm2(row_bits):
    return math.fsum(float(x) ** 2 for x in hval(row_bits))


def test_keep_selects_largest_l2_norms(orc):
    """Per block the ceil(p Bk / 100) tokens of largest exact squared L2 norm (ties to
    the lower token) are kept, in ascending order, with their exact rows.  The block
    plants a tie among the top norms and a token whose L1 norm is large but whose L2
    norm is not."""
    rng = np.random.default_rng(61)
    D, Bk, T = 16, 16, 48
    c = tiny(head_dim=D, k_block=Bk, tokens=T, v_group=D, keep_pct=15)    # 2.4 -> 3 per block
    x = rng.standard_normal((T, D))
    x[3] = 4.0                   # block 0: tokens 3 and 9 tie at the top
    x[9] = x[3]
    for j, a in ((17, 15.0), (22, 15.5), (27, 16.0)):     # block 1: one large element each:
        x[j] = 0.0                                        # L2^2 225 to 256, L1 15 to 16
        x[j, 5] = a
    x[20] = 3.5                  # L1 56 (largest by L1), L2^2 196: not kept
    k = f16(x)
    v = f16(rng.standard_normal((T, D)))
    assert orc.keep_count(c) == 3
    hc = orc.HeadCache(c).build(k, v)
    for n in range(T // Bk):
        norms = [_exact_norm2(k[n * Bk + j]) for j in range(Bk)]
        order = sorted(range(Bk), key=lambda j: (-norms[j], j))[:3]
        want = sorted(order)
        got = list(hc.k_keep_idx[n * 3:(n + 1) * 3])
        assert got == want, (n, got, want)
        for r, j in enumerate(want):
            assert np.array_equal(hc.k_keep_val[n * 3 + r], k[n * Bk + j])
    assert 3 in hc.k_keep_idx[:3] and 9 in hc.k_keep_idx[:3]           # the tie: both fit
    assert list(hc.k_keep_idx[3:6]) == [1, 6, 11]                      # offsets in block 1


def test_keep_tie_goes_to_the_lower_token(orc):
    rng = np.random.default_rng(62)
    D, Bk = 16, 16
    c = tiny(head_dim=D, k_block=Bk, tokens=Bk, v_group=D, keep_pct=5)     # 0.8 -> 1
    x = rng.standard_normal((Bk, D)) * 0.1
    x[6] = 2.0
    x[11] = 2.0
    hc = orc.HeadCache(c).build(f16(x), f16(x))
    assert list(hc.k_keep_idx) == [6]


def test_kept_rows_leave_the_statistics(orc):
    """A kept token takes no part in its block's per-channel statistics: the block's
    scale, zero and the other tokens' codes equal those of the same block with the kept
    row replaced by a copy of a neighbour (which changes no minimum or maximum) and
    nothing kept."""
    rng = np.random.default_rng(63)
    D, Bk = 16, 16
    x = rng.standard_normal((Bk, D))
    x[5] *= 9.0
    c = tiny(head_dim=D, k_block=Bk, tokens=Bk, v_group=D, keep_pct=5)
    a = orc.HeadCache(c).build(f16(x), f16(x))
    assert list(a.k_keep_idx) == [5]
    y = x.copy()
    y[5] = y[4]
    b = orc.HeadCache(tiny(head_dim=D, k_block=Bk, tokens=Bk, v_group=D)).build(f16(y), f16(x))
    assert np.array_equal(a.k_scale, b.k_scale) and np.array_equal(a.k_zero, b.k_zero)
    ka, kb_ = _deq(a, 0), _deq(b, 0)
    rows = [j for j in range(Bk) if j != 5]
    assert np.array_equal(ka[rows], kb_[rows])
    assert np.array_equal(ka[5], hval(f16(x[5])))                        # read exactly


def test_kept_keys_are_exact_in_textbook_attention(orc):
    """On-grid keys plus, in every block, two off-grid keys of much larger norm: with two
    keys kept per block the cache dequantizes exactly, so the decode equals plain fp64
    softmax attention with rotary matrices on the raw inputs; without keeping it does
    not."""
    rng = np.random.default_rng(64)
    D, Bk, T = 16, 16, 48
    L = 15
    k = _on_grid(rng, T, D, Bk, L, True)
    for n in range(T // Bk):
        for j in (n * Bk + 2, n * Bk + 13):
            k[j] = rng.standard_normal(D) * 8.0 + 20.0
    v = _on_grid(rng, T, D, Bk, L, False)
    kb, vb = f16(k), f16(v)
    c = tiny(head_dim=D, k_block=Bk, tokens=T, v_group=D, keep_pct=10)   # 1.6 -> 2
    hc = orc.HeadCache(c).build(kb, vb)
    assert np.array_equal(_deq(hc, 0), hval(kb))
    q = f16(rng.standard_normal(D))
    qp = T - 1
    qr = _rot_matrix(qp, D, 10000.0) @ hval(q)
    kr = np.stack([_rot_matrix(t, D, 10000.0) @ hval(kb[t]) for t in range(T)])
    ref = _softmax_attn(qr, kr, hval(vb), D)
    assert np.max(np.abs(hc.decode(q, q_pos=qp) - ref)) < 1e-12
    plain = orc.HeadCache(tiny(head_dim=D, k_block=Bk, tokens=T, v_group=D)).build(kb, vb)
    assert np.max(np.abs(plain.decode(q, q_pos=qp) - ref)) > 1e-6


def test_keep_layout_sizes(orc):
    c = tiny(head_dim=16, k_block=16, tokens=64, v_group=16, keep_pct=15, batch=2, kv_heads=3, q_heads=3)
    lay = orc.layout(c)
    assert lay["k_keep_idx"] == 2 * 3 * 4 * 3 and lay["k_keep_val"] == 2 * 3 * 4 * 3 * 16 * 2
    assert orc.layout(tiny())["k_keep_idx"] == 0


# --------------------------------------------------------------------------- codebook values
def _vlut_cfg(D=16, vb=2, Bk=16, T=48, **kw):
    return tiny(head_dim=D, k_block=Bk, tokens=T, k_bits=4, v_bits=vb, v_group=D, v_mode=1, **kw)


def test_value_codebook_codes_are_nearest_centroid(orc):
    """Values quantized by a per-channel sorted codebook: every dequantized value is
    the nearest entry of its channel (brute force over the entries), whatever the key
    width (keys 4-bit, values 2-bit here)."""
    rng = np.random.default_rng(71)
    c = _vlut_cfg()
    vlut = np.sort(rng.standard_normal((16, 4)) * 1.2, axis=1).astype(np.float16).view(np.uint16)
    k = _rand_block(rng, 48, 16)
    v = _rand_block(rng, 48, 16)
    hc = orc.HeadCache(c, None, vlut).build(k, v)
    x = hval(v)
    xh = _deq(hc, 1)
    C = hval(vlut)                                              # [D][4]
    best = np.argmin(np.abs(x[:, :, None] - C[None]), axis=2)
    got = np.argmax(xh[:, :, None] == C[None], axis=2)
    mids = (C[:, :-1] + C[:, 1:]) / 2
    near = np.min(np.abs(x[:, :, None] - mids[None]), axis=2) < 1e-6 * (1 + np.abs(x))
    assert np.array_equal(best[~near], got[~near])
    assert np.all(np.isin(xh, C))
    # keys are still uniform and their codes unaffected by the value codebook
    ref = orc.HeadCache(tiny(head_dim=16, k_block=16, tokens=48, v_group=16)).build(k, v)
    assert np.array_equal(_deq(hc, 0), _deq(ref, 0))


def test_value_codebook_ties_go_to_the_lower_entry(orc):
    rng = np.random.default_rng(72)
    c = _vlut_cfg(vb=4)
    z, s = -1.0, 0.125
    vlut = np.tile(f16(z + s * np.arange(16)), (16, 1))
    v = _rand_block(rng, 48, 16, scale=0.5)
    v[5] = f16(z + s * (np.arange(16) % 15 + 0.5))              # exact midpoints
    hc = orc.HeadCache(c, None, vlut).build(v, v)
    u = (hval(v) - z) / s
    want = np.clip(np.floor(u + 0.5 - 1e-12), 0, 15)
    got = (_deq(hc, 1) - z) / s
    assert np.array_equal(got, want)


def test_log_spaced_codebook_keeps_its_levels_and_is_finer_near_zero(orc):
    """Log quantization as a codebook: levels +-s 2^-k.  Values on a level come back
    exactly; the step between neighbouring levels halves towards zero."""
    import synth
    rng = np.random.default_rng(73)
    c = _vlut_cfg(vb=4)
    lut = synth.log_vlut(dict(c, kv_heads=1), np.full((1, 16), 3.0))[0]      # [D][16]
    C = hval(lut)
    assert np.all(np.diff(C, axis=1) > 0)
    pos = C[0][C[0] > 0]
    assert np.allclose(pos / pos.max(), 2.0 ** -np.arange(len(pos))[::-1])
    steps = np.diff(pos)
    assert np.allclose(steps[1:] / steps[:-1], 2.0)
    idx = rng.integers(0, 16, (48, 16))
    v = np.take_along_axis(np.broadcast_to(lut, (48, 16, 16)), idx[:, :, None], axis=2)[:, :, 0]
    hc = orc.HeadCache(c, None, lut).build(_rand_block(rng, 48, 16), v)
    assert np.array_equal(_deq(hc, 1), hval(v))


def test_codebook_values_are_exact_in_textbook_attention(orc):
    """Keys on their block grid and values on their channel's codebook: the cache
    dequantizes exactly, so the decode equals plain fp64 softmax attention with rotary
    matrices on the raw inputs."""
    rng = np.random.default_rng(74)
    D, Bk, T = 16, 16, 48
    k = f16(_on_grid(rng, T, D, Bk, 15, True))
    vlut = np.sort(rng.standard_normal((D, 4)) * 2.0, axis=1).astype(np.float16).view(np.uint16)
    idx = rng.integers(0, 4, (T, D))
    v = np.take_along_axis(np.broadcast_to(vlut, (T, D, 4)), idx[:, :, None], axis=2)[:, :, 0]
    c = _vlut_cfg(D=D, Bk=Bk, T=T)
    hc = orc.HeadCache(c, None, vlut).build(k, v)
    assert np.array_equal(_deq(hc, 1), hval(v))
    q = f16(rng.standard_normal(D))
    for qp in (T - 1, 5):
        qr = _rot_matrix(qp, D, 10000.0) @ hval(q)
        kr = np.stack([_rot_matrix(t, D, 10000.0) @ hval(k[t]) for t in range(T)])
        ref = _softmax_attn(qr, kr, hval(v), D)
        assert np.max(np.abs(hc.decode(q, q_pos=qp) - ref)) < 1e-12


def test_value_codebook_layout_sizes(orc):
    c = _vlut_cfg(D=16, vb=2, T=64, batch=2, kv_heads=3, q_heads=3)
    lay = orc.layout(c)
    assert lay["v_scale"] == 0 and lay["v_zero"] == 0
    assert lay["v_lut"] == 3 * 16 * 4 * 2
    assert lay["v_codes"] == 2 * 3 * 64 * 16 * 2 // 8
    assert orc.layout(tiny())["v_lut"] == 0


# --------------------------------------------------------------------------- FP8 cache
def _fp8_cfg(D=16, Bk=16, T=48, **kw):
    return tiny(head_dim=D, k_block=Bk, tokens=T, k_bits=8, k_mode=2, v_bits=8, v_mode=2, v_group=D, **kw)


def test_e4m3_conversion_matches_torch_cast(orc):
    """Every fp16 value: the oracle's E4M3 cast (nearest, ties to even) equals torch's
    float8_e4m3fn cast, which overflows to NaN where the oracle saturates: compared on
    the value clamped to +-448.  Infinities saturate, NaN stays NaN."""
    import torch
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = orc.e4m3_from_f16(h)
    f = torch.from_numpy(h.view(np.int16)).view(torch.float16).to(torch.float32)
    ref = f.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    fin = torch.isfinite(f).numpy()
    assert np.array_equal(mine[fin], ref[fin])
    assert orc.e4m3_from_f16(np.uint16(0x7C00)) == 0x7E and orc.e4m3_from_f16(np.uint16(0xFC00)) == 0xFE
    assert (orc.e4m3_from_f16(np.uint16(0x7E00)) & 0x7F) == 0x7F
    assert orc.e4m3_from_f16(f16(464.0)) == 0x7E and orc.e4m3_from_f16(f16(1.0625)) == 0x38    # ties to even


def test_e4m3_decode_matches_torch(orc):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    back = orc.e4m3_to_f(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    same = (back == ref) | (np.isnan(back) & np.isnan(ref))
    assert same.all()
    assert np.nanmax(np.abs(back)) == 448.0 and np.isnan(back[0x7F]) and back[1] == 2.0 ** -9


def test_fp8_cache_dequantizes_to_the_cast(orc):
    """Keys and values of an FP8 cache read back as the E4M3 cast of their input, in
    quantized blocks and (exactly) in the fp16 tail."""
    import torch
    rng = np.random.default_rng(81)
    c = _fp8_cfg(T=53)
    k = f16(rng.standard_normal((53, 16)) * 40.0)
    v = f16(rng.standard_normal((53, 16)) * 3.0)
    hc = orc.HeadCache(c).build(k, v)
    nq = 48
    for which, x in ((0, k), (1, v)):
        cast = torch.from_numpy(x[:nq].view(np.int16)).view(torch.float16).to(torch.float32).clamp(-448, 448)
        want = cast.to(torch.float8_e4m3fn).to(torch.float32).numpy()
        got = _deq(hc, which)
        assert np.array_equal(got[:nq], want)
        assert np.array_equal(got[nq:], hval(x[nq:]))


def test_fp8_cache_is_exact_in_textbook_attention(orc):
    """Keys and values that are E4M3 numbers come back exactly, so the decode equals
    plain fp64 softmax attention with rotary matrices on the raw inputs."""
    rng = np.random.default_rng(82)
    D, Bk, T = 16, 16, 48
    codes = rng.integers(0, 256, (2, T, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                        # no NaN
    kv = orc.e4m3_to_f(codes)
    k, v = f16(kv[0]), f16(kv[1])
    hc = orc.HeadCache(_fp8_cfg(D=D, Bk=Bk, T=T)).build(k, v)
    assert np.array_equal(_deq(hc, 0), hval(k)) and np.array_equal(_deq(hc, 1), hval(v))
    q = f16(rng.standard_normal(D) * 0.02)
    for qp in (T - 1, 3):
        qr = _rot_matrix(qp, D, 10000.0) @ hval(q)
        kr = np.stack([_rot_matrix(t, D, 10000.0) @ hval(k[t]) for t in range(T)])
        ref = _softmax_attn(qr, kr, hval(v), D)
        assert np.max(np.abs(hc.decode(q, q_pos=qp) - ref)) < 1e-9 * max(1.0, np.abs(ref).max())


def test_fp8_layout_sizes(orc):
    lay = orc.layout(_fp8_cfg(T=64, batch=2, kv_heads=3, q_heads=3))
    assert lay["k_codes"] == lay["v_codes"] == 2 * 3 * 64 * 16          # one byte per element
    assert lay["k_scale"] == lay["k_zero"] == lay["v_scale"] == lay["v_zero"] == 0
    assert lay["k_lut"] == lay["v_lut"] == 0
