"""Planted mistakes: each entry below patches one plausible error into a private
copy of oracle.c (a dropped term, a wrong sign, index or rounding direction), and
the pins in test_oracle_pins.py must reject every one of them.  CPU only; the
mutated builds live in a temporary directory."""
import inspect
import os

import pytest

import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

MUTANTS = {
    "rope_direction": ("y[i] = a * cs - b * sn;", "y[i] = a * cs + b * sn;"),
    "rope_frequency": ("pow(theta, -(2.0 * i) / (double)D)", "pow(theta, -(1.0 * i) / (double)D)"),
    "dropped_inv_sqrt_d": ("s[t] = acc * inv_sqrt_d;", "s[t] = acc;"),
    "zero_round_nearest": ("*z16 = orc_f2h_rd(lo);", "*z16 = orc_f2h_rn(lo);"),
    "scale_round_nearest": ("*s16 = orc_f2h_ru(s32);", "*s16 = orc_f2h_rn(s32);"),
    "scale_uses_L_plus_1": ("const float s32 = range / (float)L;", "const float s32 = range / (float)(L + 1);"),
    "outlier_tie_higher_column": ("(row[d] & 0x7fff) > (row[best] & 0x7fff)", "(row[d] & 0x7fff) >= (row[best] & 0x7fff)"),
    "outliers_in_key_stats": ("        if (mask[i]) continue;\n        lo = fminf(lo, d[i]);\n        hi = fmaxf(hi, d[i]);\n        ++cnt;\n      }\n      uint16_t z16, s16;\n      orc_meta(lo, hi, cnt, L, &z16, &s16);\n      hd->k_scale",
                              "        lo = fminf(lo, d[i]);\n        hi = fmaxf(hi, d[i]);\n        ++cnt;\n      }\n      uint16_t z16, s16;\n      orc_meta(lo, hi, cnt, L, &z16, &s16);\n      hd->k_scale"),
    "kout_floor": ("(c->outlier_pct * c->head_dim + 99) / 100", "(c->outlier_pct * c->head_dim) / 100"),
    "clip_no_interpolation": ("const double f = pos - (double)k;", "const double f = 0.0;"),
    "clip_one_sided": ("d[i] = clip ? fminf(fmaxf(x, -thr), thr) : x;", "d[i] = clip ? fminf(x, thr) : x;"),
    "round_half_up": ("float r = nearbyintf(q);", "float r = floorf(q + 0.5f);"),
    "dequant_drops_zero": ("out[ch] = fmaf((float)cc, orc_h2f(hd->v_scale[t * ng + ch / G]),\n                       orc_h2f(hd->v_zero[t * ng + ch / G]));",
                           "out[ch] = (float)cc * orc_h2f(hd->v_scale[t * ng + ch / G]);"),
    "key_natural_order": ("return (e >> 1) + (e & 1) * (D / 2);", "return e;"),
    "value_word_transposed": ("return ((t / tpw) * (int64_t)c->head_dim + d) * 32 + (t % tpw) * c->v_bits;",
                              "return ((int64_t)d * (c->capacity / tpw) + t / tpw) * 32 + (t % tpw) * c->v_bits;"),
    "lut_ties_upper": ("cc += d[i] > mid[k];", "cc += d[i] >= mid[k];"),
    "softmax_uses_key_as_value": ("orc_dequant_row(c, hd, 1, t, row);", "orc_dequant_row(c, hd, 0, t, row);"),
    "f2h_truncates": ("float r = nearbyintf(ldexpf(a, 10 - e));", "float r = truncf(ldexpf(a, 10 - e));"),
    "chunk_excludes_own_token": ("int64_t nvis = q_pos + j + 1;", "int64_t nvis = q_pos + j;"),
    "chunk_sees_whole_cache": ("if (nvis > hd->length) nvis = hd->length;", "nvis = hd->length;"),
    "chunk_rotates_all_rows_at_first_position": ("q_pos + j, nvis,", "q_pos, nvis,"),
    "chunk_row_offset_ignored": ("out + (int64_t)j * c->head_dim))", "out))"),
    "keep_smallest_norm": ("if (best < 0 || norm[j] > norm[best]) best = j;",
                           "if (best < 0 || norm[j] < norm[best]) best = j;"),
    "keep_tie_higher_token": ("if (best < 0 || norm[j] > norm[best]) best = j;",
                              "if (best < 0 || norm[j] >= norm[best]) best = j;"),
    "keep_norm_l1": ("    s += x * x;", "    s += fabs(x);"),
    "kept_rows_in_stats": ("    memset(mask + (int64_t)j * D, 1, (size_t)D);\n", ""),
    "kept_key_read_quantized": ("out[ch] = orc_h2f(hd->k_keep_val[(n * R + r) * D + ch]);", "out[ch] = out[ch];"),
    "keep_count_floor": ("(c->keep_pct * c->k_block + 99) / 100", "(c->keep_pct * c->k_block) / 100"),
    # (mistakes that stay inside the buffers: the mutated oracle runs in this process)
    "vlut_row_stride_halved": ("orc_h2f(hd->v_lut[(int64_t)ch * (1 << c->v_bits) + cc])",
                               "orc_h2f(hd->v_lut[(int64_t)ch * (1 << (c->v_bits - 1)) + cc])"),
    "vlut_channel_ignored": ("orc_h2f(hd->v_lut[(int64_t)ch * (1 << c->v_bits) + cc])", "orc_h2f(hd->v_lut[cc])"),
    "e4m3_ties_away": ("float q = nearbyintf(ldexpf(a, 3 - ex));", "float q = roundf(ldexpf(a, 3 - ex));"),
    "e4m3_overflow_to_nan": ("if (r > 448.0f) return (uint8_t)(sign | 0x7E);", "if (r > 448.0f) return (uint8_t)(sign | 0x7F);"),
    "e4m3_bias_8": ("return (uint8_t)(sign | (uint8_t)((ex + 7) << 3) | (uint8_t)((int)q - 8));",
                    "return (uint8_t)(sign | (uint8_t)((ex + 8) << 3) | (uint8_t)((int)q - 8));"),
    "e4m3_decode_bias_off_by_one": ("v = ldexpf((float)(8 + m), e - 10);", "v = ldexpf((float)(8 + m), e - 11);"),
    "vlut_not_in_layout": ("out[17] = c->v_mode == 1 ? (int64_t)c->kv_heads * D * (1 << c->v_bits) * 2 : 0;",
                           "out[17] = 0;"),
}


def _pin_tests():
    """Every pin test with its parametrisations, as (name, callable)."""
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        combos = [dict()]
        for m in params:
            argnames = [a.strip() for a in (m.args[0].split(",") if isinstance(m.args[0], str) else m.args[0])]
            new = []
            for base in combos:
                for val in m.args[1]:
                    vals = val if len(argnames) > 1 else (val,)
                    d = dict(base)
                    d.update(zip(argnames, vals))
                    new.append(d)
            combos = new
        for kw in combos:
            out.append((name, fn, kw))
    return out


def test_every_mutant_source_patch_applies():
    src = open(SRC).read()
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, name


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_reject_planted_mistake(orc, tmp_path, mutant):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) == 1
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = orc.compile_source(str(path), str(tmp_path / "libmutant.so"))
    caught = []
    orc.use_library(so)
    try:
        for name, fn, kw in _pin_tests():
            try:
                fn(orc, **kw) if "orc" in inspect.signature(fn).parameters else fn(**kw)
            except (AssertionError, RuntimeError, ValueError, IndexError):
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, "no pin rejects the planted mistake %r" % mutant
