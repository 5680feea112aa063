/*
 * oracle.c -- plain, slow, scalar CPU oracle for low-bit KV-cache quantization
 * and decode attention over the quantized cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library.  It shares no source, header,
 * table or helper with the HIP library; the two meet only through the seeded
 * inputs drawn by the `synth` package.
 *
 * Pages cited (title, address):
 *   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
 *   [TQ]   "TurboQuant：突破大模型推理瓶颈的KVCache量化技术解析", mlqm.cn/news/1002276
 *   [UQ]   "大模型长上下文推理优化：4-bit KV Cache量化技术解析与部署实践", mlqm.cn/news/1064729
 *
 * Arithmetic: the quantizer works in fp32 with every operation rounded
 * separately (build with -O2 -ffp-contract=off, no fast-math), round-half-to-even;
 * the attention works in fp64 over the fp32 dequantized values.
 *
 * Functions whose result has no outside pin are marked "parity unpinned"; at the
 * time of writing there are none: every function here is pinned by a test in
 * tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Same fields, same meaning as the library's configuration (defined independently). */
typedef struct {
  int32_t batch, q_heads, kv_heads, head_dim, capacity;
  int32_t k_bits, k_mode, k_block;
  int32_t v_bits, v_group;
  float clip_quantile;
  int32_t outlier_pct;
  float rope_theta;
  int32_t keep_pct;        /* key vectors kept in fp16 per block, percent (0 = none) */
  int32_t v_mode;          /* 0: uniform per-token values; 1: per-channel codebook;    */
                           /* 2: fp8 e4m3 (with k_mode 2)                             */
} orc_cfg;

/* Buffers of ONE (batch, kv-head) of the cache, laid out exactly as the library's
 * per-(b, h) slices. */
typedef struct {
  uint8_t *k_codes;        /* [capacity][D*k_bits/8]                          */
  uint16_t *k_scale;       /* [capacity/k_block][D]  fp16 (uniform keys)       */
  uint16_t *k_zero;        /* [capacity/k_block][D]  fp16 (uniform keys)       */
  const uint16_t *k_lut;   /* [D][2^k_bits]          fp16 (codebook keys)      */
  uint16_t *k_tail;        /* [k_block][D]           fp16                      */
  uint8_t *v_codes;        /* capacity*D*v_bits/8 bytes, token-group words     */
  uint16_t *v_scale;       /* [capacity][D/v_group]  fp16                      */
  uint16_t *v_zero;        /* [capacity][D/v_group]  fp16                      */
  uint16_t *v_tail;        /* [k_block][D]           fp16                      */
  int32_t *k_rowptr;       /* [capacity+1]                                      */
  uint8_t *k_col;          /* [capacity*k_out]                                  */
  uint16_t *k_val;         /* [capacity*k_out]       fp16                      */
  int32_t *v_rowptr;
  uint8_t *v_col;
  uint16_t *v_val;
  uint8_t *k_keep_idx;     /* [capacity/k_block][R]    retained token offsets      */
  uint16_t *k_keep_val;    /* [capacity/k_block][R][D] their keys, fp16           */
  const uint16_t *v_lut;   /* [D][2^v_bits]          fp16 (codebook values)    */
  int64_t length;          /* tokens held                                       */
} orc_head;

/* ------------------------------------------------------------------------- */
/* fp16 <-> fp32, written out from the IEEE binary16 definition.              */
/* ------------------------------------------------------------------------- */

float orc_h2f(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int m = h & 0x3ff;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -24);                    /* zero and subnormals */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexpf((float)(m | 0x400), e - 25);       /* (1024 + m) * 2^(e-25) */
  return sign ? -v : v;
}

/* round to nearest, ties to even */
/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN, so the largest finite value is 1.75 * 2^8 = 448; the
 * smallest normal 2^-6, subnormals m * 2^-9.  Written from that definition. */
float orc_e4m3_to_f(uint8_t b) {
  const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
  float v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexpf((float)m, -9);
  else
    v = ldexpf((float)(8 + m), e - 10);           /* (8 + m) * 2^(e-7-3) */
  return sign ? -v : v;
}

/* fp16 -> E4M3, round to nearest, ties to even; magnitudes beyond the largest finite
 * value (infinities included) saturate to +-448; NaN gives S.1111.111.  The fp16
 * value is exact in float; the grid step at |x| is 2^(floor(log2|x|) - 3) for normal
 * results and 2^-9 below 2^-6, and nearbyintf rounds ties to even. */
uint8_t orc_f_to_e4m3(uint16_t h) {
  const float x = orc_h2f(h);
  const uint8_t sign = (uint8_t)((h >> 15) << 7);
  if (x != x) return (uint8_t)(sign | 0x7F);
  float a = fabsf(x);
  if (a == 0.0f) return sign;
  if (isinf(a)) return (uint8_t)(sign | 0x7E);      /* saturate */
  int e;
  (void)frexpf(a, &e);                              /* a = f * 2^e, f in [0.5, 1) */
  int ex = e - 1;                                   /* floor(log2 a) */
  if (ex < -6) ex = -6;                             /* subnormal step 2^-9 */
  float q = nearbyintf(ldexpf(a, 3 - ex));          /* units of 2^(ex-3) */
  if (q >= 16.0f) { q = 8.0f; ex += 1; }            /* rounded up to the next binade */
  const float r = ldexpf(q, ex - 3);
  if (r > 448.0f) return (uint8_t)(sign | 0x7E);    /* saturate */
  if (ex == -6 && q < 8.0f) return (uint8_t)(sign | (uint8_t)q);              /* subnormal */
  return (uint8_t)(sign | (uint8_t)((ex + 7) << 3) | (uint8_t)((int)q - 8));  /* normal */
}

uint16_t orc_f2h_rn(float f) {
  const uint16_t sign = signbit(f) ? 0x8000 : 0;
  const float a = fabsf(f);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00);
  if (isinf(f)) return (uint16_t)(sign | 0x7c00);
  if (a < 0x1p-14f) {                              /* subnormal binade: step 2^-24 */
    const float r = nearbyintf(a * 0x1p24f);        /* exact scaling, then RNE */
    return (uint16_t)(sign | (uint16_t)r);          /* r == 1024 is the smallest normal */
  }
  int e;
  frexpf(a, &e);
  e -= 1;                                           /* a = m * 2^e with m in [1, 2) */
  float r = nearbyintf(ldexpf(a, 10 - e));          /* mantissa with 10 fraction bits */
  uint32_t m = (uint32_t)r;
  if (m == 2048) { m = 1024; e += 1; }
  if (e > 15) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | (m - 1024));
}

static uint16_t orc_h_next_down(uint16_t h) {
  if ((h & 0x7fff) == 0) return 0x8001;
  return (h & 0x8000) ? (uint16_t)(h + 1) : (uint16_t)(h - 1);
}
static uint16_t orc_h_next_up(uint16_t h) {
  if ((h & 0x7fff) == 0) return 0x0001;
  return (h & 0x8000) ? (uint16_t)(h - 1) : (uint16_t)(h + 1);
}
/* largest fp16 <= v */
uint16_t orc_f2h_rd(float v) {
  uint16_t h = orc_f2h_rn(v);
  if (orc_h2f(h) > v) h = orc_h_next_down(h);
  return h;
}
/* smallest fp16 >= v */
uint16_t orc_f2h_ru(float v) {
  uint16_t h = orc_f2h_rn(v);
  if (orc_h2f(h) < v) h = orc_h_next_up(h);
  return h;
}

void orc_h2f_array(const uint16_t *h, float *f, int64_t n) {
  for (int64_t i = 0; i < n; ++i) f[i] = orc_h2f(h[i]);
}
void orc_f2h_array(const float *f, uint16_t *h, int64_t n, int mode /*0 rn, 1 rd, 2 ru*/) {
  for (int64_t i = 0; i < n; ++i)
    h[i] = mode == 0 ? orc_f2h_rn(f[i]) : mode == 1 ? orc_f2h_rd(f[i]) : orc_f2h_ru(f[i]);
}

/* ------------------------------------------------------------------------- */
/* Sizes.                                                                     */
/* ------------------------------------------------------------------------- */

/* KV-cache bytes = 2 (K and V) x layers x batch x tokens x hidden x bytes per
 * element: the size formula of [TQ] section 2.1, with bytes given in bits. */
double orc_kv_bytes(int64_t layers, int64_t batch, int64_t tokens, int64_t hidden,
                    int64_t bits_per_elem) {
  return 2.0 * (double)layers * (double)batch * (double)tokens * (double)hidden *
         (double)bits_per_elem / 8.0;
}

int orc_kout(const orc_cfg *c) {
  return c->outlier_pct > 0 ? (c->outlier_pct * c->head_dim + 99) / 100 : 0;
}

/* Key vectors kept in fp16 per quantized block: ceil(keep_pct * k_block / 100). */
int orc_keep_count(const orc_cfg *c) {
  return c->keep_pct > 0 ? (c->keep_pct * c->k_block + 99) / 100 : 0;
}

/* Byte size of every buffer of the whole cache, in the order
 * k_codes k_scale k_zero k_lut k_tail v_codes v_scale v_zero v_tail
 * k_rowptr k_col k_val v_rowptr v_col v_val k_keep_idx k_keep_val v_lut (18 entries). */
void orc_layout(const orc_cfg *c, int64_t out[18]) {
  const int64_t BH = (int64_t)c->batch * c->kv_heads, D = c->head_dim, T = c->capacity;
  const int64_t nblk = T / c->k_block, ko = orc_kout(c);
  const int uni = c->k_mode == 0;
  out[0] = BH * T * D * c->k_bits / 8;
  out[1] = uni ? BH * nblk * D * 2 : 0;
  out[2] = out[1];
  out[3] = c->k_mode == 1 ? (int64_t)c->kv_heads * D * (1 << c->k_bits) * 2 : 0;
  out[4] = BH * c->k_block * D * 2;
  out[5] = BH * T * D * c->v_bits / 8;
  out[6] = c->v_mode != 0 ? 0 : BH * T * (D / c->v_group) * 2;
  out[7] = out[6];
  out[8] = out[4];
  out[9] = ko ? BH * (T + 1) * 4 : 0;
  out[10] = BH * T * ko;
  out[11] = BH * T * ko * 2;
  out[12] = out[9];
  out[13] = out[10];
  out[14] = out[11];
  out[15] = BH * nblk * orc_keep_count(c);
  out[16] = out[15] * D * 2;
  out[17] = c->v_mode == 1 ? (int64_t)c->kv_heads * D * (1 << c->v_bits) * 2 : 0;
}

/* Importance of a key vector: its squared L2 norm, the squares of the fp16 values
 * (exact in fp64) added in channel order in fp64 ([TQ] section 3.2: importance from the
 * vector's own norm; section 6.1: the L2 norm directly). */
static double orc_key_norm2(const uint16_t *row, int D) {
  double s = 0.0;
  for (int d = 0; d < D; ++d) {
    const double x = (double)orc_h2f(row[d]);
    s += x * x;
  }
  return s;
}

/* The R key vectors of a block kept in fp16 ([TQ] section 3.2: the few important keys
 * keep high precision, the rest are quantized): the R largest norms, ties to the lower
 * token; written in ascending token order; their rows are masked out of the block's
 * statistics and take code 0. */
static void orc_keep_rows(const orc_cfg *c, int64_t n, const uint16_t *src, uint8_t *mask,
                          orc_head *hd) {
  const int D = c->head_dim, Bk = c->k_block, R = orc_keep_count(c);
  double norm[256];
  uint8_t kept[256];
  int sel[64];
  for (int j = 0; j < Bk; ++j) {
    norm[j] = orc_key_norm2(src + (int64_t)j * D, D);
    kept[j] = 0;
  }
  for (int r = 0; r < R; ++r) {
    int best = -1;
    for (int j = 0; j < Bk; ++j) {
      if (kept[j]) continue;
      if (best < 0 || norm[j] > norm[best]) best = j;
    }
    kept[best] = 1;
    sel[r] = best;
  }
  for (int a = 1; a < R; ++a)
    for (int b = a; b > 0 && sel[b - 1] > sel[b]; --b) {
      int t = sel[b]; sel[b] = sel[b - 1]; sel[b - 1] = t;
    }
  for (int r = 0; r < R; ++r) {
    const int j = sel[r];
    hd->k_keep_idx[n * R + r] = (uint8_t)j;
    memcpy(hd->k_keep_val + (n * R + r) * D, src + (int64_t)j * D, (size_t)D * sizeof(uint16_t));
    memset(mask + (int64_t)j * D, 1, (size_t)D);
  }
}

/* ------------------------------------------------------------------------- */
/* Quantize one complete token block of one (b, h), K or V.                   */
/* ------------------------------------------------------------------------- */

/* Dense-and-sparse split ([KVC3] "Per-Vector Dense-and-Sparse Quantization"):
 * the k_out elements of largest |x| (ties: lower column first) are kept exactly
 * as fp16; columns are emitted in ascending order. */
static void orc_outliers_row(const uint16_t *row, int D, int kout, uint8_t *mask_row,
                             uint8_t *cols, uint16_t *vals) {
  int sel[256];
  uint8_t picked[256];
  memset(picked, 0, sizeof picked);
  for (int r = 0; r < kout; ++r) {
    int best = -1;
    for (int d = 0; d < D; ++d) {
      if (picked[d]) continue;
      /* |x| compared on the fp16 magnitude bits: for finite values their integer
       * order is the order of |x| */
      if (best < 0 || (row[d] & 0x7fff) > (row[best] & 0x7fff)) best = d;
    }
    picked[best] = 1;
    sel[r] = best;
  }
  for (int a = 1; a < kout; ++a)
    for (int b = a; b > 0 && sel[b - 1] > sel[b]; --b) {
      int t = sel[b]; sel[b] = sel[b - 1]; sel[b - 1] = t;
    }
  for (int r = 0; r < kout; ++r) {
    cols[r] = (uint8_t)sel[r];
    vals[r] = row[sel[r]];
    mask_row[sel[r]] = 1;
  }
}

static int orc_cmp_u16(const void *a, const void *b) {
  const uint16_t x = *(const uint16_t *)a, y = *(const uint16_t *)b;
  return (x > y) - (x < y);
}

/* Clip threshold: the q-quantile of |x| over the whole block, by exact order
 * statistics with linear interpolation between neighbours, like the percentile
 * clip in [UQ] section 4.2.  fp64 interpolation with the product and the sum
 * rounded separately, then rounded to fp32. */
float orc_clip_threshold(const uint16_t *blk, int64_t n, float q) {
  uint16_t *mag = (uint16_t *)malloc((size_t)n * sizeof(uint16_t));
  for (int64_t i = 0; i < n; ++i) mag[i] = blk[i] & 0x7fff;
  qsort(mag, (size_t)n, sizeof(uint16_t), orc_cmp_u16);
  const double pos = (double)q * (double)(n - 1);
  const int64_t k = (int64_t)floor(pos);
  const double f = pos - (double)k;
  const double vk = (double)orc_h2f(mag[k]);
  float t;
  if (k + 1 >= n) {
    t = (float)vk;
  } else {
    const double vk1 = (double)orc_h2f(mag[k + 1]);
    const double diff = vk1 - vk;
    const double prod = f * diff;
    const double sum = vk + prod;
    t = (float)sum;
  }
  free(mag);
  return t;
}

/* Uniform asymmetric code: c = clamp(round_half_even((d - z) / s), 0, L), with
 * the fp32 subtract and the fp32 divide each correctly rounded; c = 0 when the
 * scale is 0 (a constant or empty group).  Follows round(x/scale) of [TQ]
 * section 4.2 with the zero-point of [KVC3] "Quanto 的量化原理". */
static int orc_code_uniform(float d, uint16_t z16, uint16_t s16, int L) {
  const float s = orc_h2f(s16);
  if (s == 0.0f) return 0;
  const float num = d - orc_h2f(z16);
  const float q = num / s;
  float r = nearbyintf(q);
  if (r < 0.0f) r = 0.0f;
  if (r > (float)L) r = (float)L;
  return (int)r;
}

/* Group metadata: zero = largest fp16 <= lo, scale = smallest fp16 >= (hi - zero)/L.
 * Empty groups have lo = hi = 0; -0 is canonicalised to +0. */
static void orc_meta(float lo, float hi, int cnt, int L, uint16_t *z16, uint16_t *s16) {
  if (cnt == 0) { lo = 0.0f; hi = 0.0f; }
  lo = lo + 0.0f;
  hi = hi + 0.0f;
  *z16 = orc_f2h_rd(lo);
  const float range = hi - orc_h2f(*z16);
  const float s32 = range / (float)L;
  *s16 = orc_f2h_ru(s32);
}

/* Bit position helpers of the packed layouts. */
static int orc_k_channel_of_element(int e, int D) { return (e >> 1) + (e & 1) * (D / 2); }

static void orc_put_bits(uint8_t *base, int64_t bitpos, uint32_t v, int bits) {
  const int64_t byte = bitpos >> 3;
  const int sh = (int)(bitpos & 7);
  const uint32_t w = v << sh;
  base[byte] |= (uint8_t)(w & 0xff);
  if (sh + bits > 8) base[byte + 1] |= (uint8_t)((w >> 8) & 0xff);
}
static uint32_t orc_get_bits(const uint8_t *base, int64_t bitpos, int bits) {
  const int64_t byte = bitpos >> 3;
  const int sh = (int)(bitpos & 7);
  uint32_t w = base[byte];
  if (sh + bits > 8) w |= (uint32_t)base[byte + 1] << 8;
  return (w >> sh) & ((1u << bits) - 1u);
}

/* Key row t: element e (bits [e*kb, e*kb+kb) of the row, LSB first) holds channel
 * (e >> 1) + (e & 1) * D/2, so each rotary pair (i, i + D/2) sits side by side. */
static int64_t orc_k_bitpos(const orc_cfg *c, int64_t t, int e) {
  return t * (int64_t)c->head_dim * c->k_bits + (int64_t)e * c->k_bits;
}
/* Value code of token t, channel d: 32-bit little-endian word (t / tpw) * D + d,
 * bits [(t % tpw) * vb, ...) with tpw = 32 / vb tokens per word. */
static int64_t orc_v_bitpos(const orc_cfg *c, int64_t t, int d) {
  const int tpw = 32 / c->v_bits;
  return ((t / tpw) * (int64_t)c->head_dim + d) * 32 + (t % tpw) * c->v_bits;
}

/* Per-channel non-uniform codebook ([KVC3] "Non-Uniform KV Cache Quantization"): the
 * code of x is its nearest entry among the channel's sorted fp16 centroids, decided
 * at the fp32 midpoints, ties to the lower code; marked (outlier or kept) positions
 * get code 0.  lut: [D][L + 1]; d, mask, code: the block, [Bk][D]. */
static void orc_codebook_codes(const uint16_t *lut, int D, int L, int Bk, const float *d,
                               const uint8_t *mask, uint8_t *code) {
  for (int ch = 0; ch < D; ++ch) {
    const uint16_t *C = lut + (int64_t)ch * (L + 1);
    float mid[255];
    for (int k = 0; k < L; ++k) mid[k] = (orc_h2f(C[k]) + orc_h2f(C[k + 1])) * 0.5f;
    for (int j = 0; j < Bk; ++j) {
      const int64_t i = (int64_t)j * D + ch;
      int cc = 0;
      if (!mask[i])
        for (int k = 0; k < L; ++k) cc += d[i] > mid[k];
      code[i] = (uint8_t)cc;
    }
  }
}

int orc_quantize_block(const orc_cfg *c, int is_key, int64_t n, const uint16_t *src,
                       orc_head *hd) {
  const int D = c->head_dim, Bk = c->k_block, kout = orc_kout(c);
  const int bits = is_key ? c->k_bits : c->v_bits;
  const int L = (1 << bits) - 1;
  const int64_t t0 = n * Bk, nel = (int64_t)Bk * D;
  uint8_t *mask = (uint8_t *)calloc((size_t)nel, 1);
  float *d = (float *)malloc((size_t)nel * sizeof(float));
  uint8_t *code = (uint8_t *)calloc((size_t)nel, 1);
  if (!mask || !d || !code) { free(mask); free(d); free(code); return -1; }

  /* 1. outliers, per token vector */
  if (kout > 0) {
    int32_t *rp = is_key ? hd->k_rowptr : hd->v_rowptr;
    uint8_t *col = is_key ? hd->k_col : hd->v_col;
    uint16_t *val = is_key ? hd->k_val : hd->v_val;
    if (n == 0) rp[0] = 0;
    for (int j = 0; j < Bk; ++j) {
      orc_outliers_row(src + (int64_t)j * D, D, kout, mask + (int64_t)j * D,
                       col + (t0 + j) * kout, val + (t0 + j) * kout);
      rp[t0 + j + 1] = (int32_t)((t0 + j + 1) * kout);
    }
  }
  /* 1b. the block's important key vectors, kept in fp16 */
  if (is_key && orc_keep_count(c) > 0) orc_keep_rows(c, n, src, mask, hd);
  /* 2. clip threshold over the whole block (outliers included), 3. dense values */
  const int clip = c->clip_quantile > 0.0f;
  const float thr = clip ? orc_clip_threshold(src, nel, c->clip_quantile) : 0.0f;
  for (int64_t i = 0; i < nel; ++i) {
    const float x = orc_h2f(src[i]);
    d[i] = clip ? fminf(fmaxf(x, -thr), thr) : x;
  }
  /* 4-5. statistics, metadata, codes */
  if ((is_key && c->k_mode == 2) || (!is_key && c->v_mode == 2)) {
    /* FP8 cache ([UQ] section 2.1): every element cast to E4M3, no statistics */
    for (int64_t i = 0; i < nel; ++i) code[i] = orc_f_to_e4m3(src[i]);
  } else if (is_key && c->k_mode == 1) {
    orc_codebook_codes(hd->k_lut, D, L, Bk, d, mask, code);
  } else if (!is_key && c->v_mode == 1) {
    /* The same for values: the page names the Value cache first among the tensors a
     * uniform grid fits badly; [TQ] section 3.3 names log quantization as one such
     * non-uniform grid (a codebook whose levels are spaced by powers of two). */
    orc_codebook_codes(hd->v_lut, D, L, Bk, d, mask, code);
  } else if (is_key) {
    /* Per-channel keys over the token block ([KVC3] "Per-Channel Key Quantization",
     * quantized before RoPE per "Pre-RoPE Key Quantization"). */
    for (int ch = 0; ch < D; ++ch) {
      float lo = INFINITY, hi = -INFINITY;
      int cnt = 0;
      for (int j = 0; j < Bk; ++j) {
        const int64_t i = (int64_t)j * D + ch;
        if (mask[i]) continue;
        lo = fminf(lo, d[i]);
        hi = fmaxf(hi, d[i]);
        ++cnt;
      }
      uint16_t z16, s16;
      orc_meta(lo, hi, cnt, L, &z16, &s16);
      hd->k_scale[n * D + ch] = s16;
      hd->k_zero[n * D + ch] = z16;
      for (int j = 0; j < Bk; ++j) {
        const int64_t i = (int64_t)j * D + ch;
        code[i] = mask[i] ? 0 : (uint8_t)orc_code_uniform(d[i], z16, s16, L);
      }
    }
  } else {
    /* Values per token in channel groups, each with its scale and zero-point
     * ([KVC3] "Quanto 的量化原理"). */
    const int G = c->v_group, ng = D / G;
    for (int j = 0; j < Bk; ++j)
      for (int g = 0; g < ng; ++g) {
        float lo = INFINITY, hi = -INFINITY;
        int cnt = 0;
        for (int ch = g * G; ch < (g + 1) * G; ++ch) {
          const int64_t i = (int64_t)j * D + ch;
          if (mask[i]) continue;
          lo = fminf(lo, d[i]);
          hi = fmaxf(hi, d[i]);
          ++cnt;
        }
        uint16_t z16, s16;
        orc_meta(lo, hi, cnt, L, &z16, &s16);
        hd->v_scale[(t0 + j) * ng + g] = s16;
        hd->v_zero[(t0 + j) * ng + g] = z16;
        for (int ch = g * G; ch < (g + 1) * G; ++ch) {
          const int64_t i = (int64_t)j * D + ch;
          code[i] = mask[i] ? 0 : (uint8_t)orc_code_uniform(d[i], z16, s16, L);
        }
      }
  }
  /* 6. pack ([KVC3] "Quanto 的量化原理": 4 bits per code plus a little metadata) */
  if (is_key) {
    const int64_t rowbytes = (int64_t)D * c->k_bits / 8;
    memset(hd->k_codes + t0 * rowbytes, 0, (size_t)(Bk * rowbytes));
    for (int j = 0; j < Bk; ++j)
      for (int e = 0; e < D; ++e) {
        const int ch = orc_k_channel_of_element(e, D);
        orc_put_bits(hd->k_codes, orc_k_bitpos(c, t0 + j, e), code[(int64_t)j * D + ch], bits);
      }
  } else {
    const int64_t blkbytes = (int64_t)Bk * D * c->v_bits / 8;
    memset(hd->v_codes + t0 * (int64_t)D * c->v_bits / 8, 0, (size_t)blkbytes);
    for (int j = 0; j < Bk; ++j)
      for (int ch = 0; ch < D; ++ch)
        orc_put_bits(hd->v_codes, orc_v_bitpos(c, t0 + j, ch), code[(int64_t)j * D + ch], bits);
  }
  free(mask);
  free(d);
  free(code);
  return 0;
}

/* Fill an empty head with T tokens: every complete block of k_block tokens is
 * quantized, the remainder stays as fp16 in the tail (blocks are quantized once
 * full, as in the block accumulation of [UQ] section 4.2). */
int orc_build_head(const orc_cfg *c, orc_head *hd, const uint16_t *k_src, const uint16_t *v_src,
                   int64_t T) {
  const int D = c->head_dim, Bk = c->k_block;
  if (T > c->capacity) return -1;
  const int64_t nfull = T / Bk;
  for (int64_t n = 0; n < nfull; ++n) {
    if (orc_quantize_block(c, 1, n, k_src + n * Bk * D, hd)) return -1;
    if (orc_quantize_block(c, 0, n, v_src + n * Bk * D, hd)) return -1;
  }
  const int64_t rem = T - nfull * Bk;
  memcpy(hd->k_tail, k_src + nfull * Bk * D, (size_t)(rem * D) * sizeof(uint16_t));
  memcpy(hd->v_tail, v_src + nfull * Bk * D, (size_t)(rem * D) * sizeof(uint16_t));
  hd->length = T;
  return 0;
}

int orc_build_heads(const orc_cfg *c, int64_t nheads, orc_head *hds, const uint16_t *k_src,
                    const uint16_t *v_src, int64_t T) {
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int64_t i = 0; i < nheads; ++i)
    err |= orc_build_head(c, &hds[i], k_src + i * T * c->head_dim, v_src + i * T * c->head_dim, T) != 0;
  return err ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* Dequantize.                                                                */
/* ------------------------------------------------------------------------- */

/* One token row of K (which = 0) or V (which = 1), fp32, pre-RoPE: x = fmaf(c, s, z)
 * or the codebook entry; outlier positions take their exact fp16 value; tail
 * tokens are exact. */
static void orc_dequant_row(const orc_cfg *c, const orc_head *hd, int which, int64_t t, float *out) {
  const int D = c->head_dim, Bk = c->k_block, kout = orc_kout(c);
  const int64_t nfull = (hd->length / Bk) * Bk;
  if (t >= nfull) {
    const uint16_t *tail = which ? hd->v_tail : hd->k_tail;
    for (int ch = 0; ch < D; ++ch) out[ch] = orc_h2f(tail[(t - nfull) * D + ch]);
    return;
  }
  if (which == 0) {
    const int kb = c->k_bits;
    for (int e = 0; e < D; ++e) {
      const int ch = orc_k_channel_of_element(e, D);
      const uint32_t cc = orc_get_bits(hd->k_codes, orc_k_bitpos(c, t, e), kb);
      if (c->k_mode == 2)
        out[ch] = orc_e4m3_to_f((uint8_t)cc);
      else if (c->k_mode == 1)
        out[ch] = orc_h2f(hd->k_lut[(int64_t)ch * (1 << kb) + cc]);
      else
        out[ch] = fmaf((float)cc, orc_h2f(hd->k_scale[(t / Bk) * D + ch]),
                       orc_h2f(hd->k_zero[(t / Bk) * D + ch]));
    }
  } else {
    const int G = c->v_group, ng = D / G;
    for (int ch = 0; ch < D; ++ch) {
      const uint32_t cc = orc_get_bits(hd->v_codes, orc_v_bitpos(c, t, ch), c->v_bits);
      if (c->v_mode == 2)
        out[ch] = orc_e4m3_to_f((uint8_t)cc);
      else if (c->v_mode == 1)
        out[ch] = orc_h2f(hd->v_lut[(int64_t)ch * (1 << c->v_bits) + cc]);
      else
        out[ch] = fmaf((float)cc, orc_h2f(hd->v_scale[t * ng + ch / G]),
                       orc_h2f(hd->v_zero[t * ng + ch / G]));
    }
  }
  if (kout > 0) {
    const uint8_t *col = which ? hd->v_col : hd->k_col;
    const uint16_t *val = which ? hd->v_val : hd->k_val;
    const int32_t *rp = which ? hd->v_rowptr : hd->k_rowptr;
    for (int32_t r = rp[t]; r < rp[t + 1]; ++r) out[col[r]] = orc_h2f(val[r]);
  }
  const int R = orc_keep_count(c);
  if (which == 0 && R > 0) {  /* a key kept in fp16 is read exactly */
    const int64_t n = t / Bk;
    for (int r = 0; r < R; ++r)
      if (hd->k_keep_idx[n * R + r] == (uint8_t)(t % Bk))
        for (int ch = 0; ch < D; ++ch) out[ch] = orc_h2f(hd->k_keep_val[(n * R + r) * D + ch]);
  }
}

int orc_dequantize_head(const orc_cfg *c, const orc_head *hd, int which, int64_t t0, int64_t t1,
                        float *out) {
  if (t0 < 0 || t1 > hd->length || t0 > t1) return -1;
  for (int64_t t = t0; t < t1; ++t) orc_dequant_row(c, hd, which, t, out + (t - t0) * c->head_dim);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Decode attention, fp64.                                                    */
/* ------------------------------------------------------------------------- */

/* Rotary embedding, rotate-half convention: channel pair (i, i + D/2) turns by
 * pos * theta^(-2i/D).  Keys are rotated after dequantization ([KVC3]
 * "Pre-RoPE Key Quantization"). */
static void orc_rope(const double *x, double *y, int D, double pos, double theta) {
  const int half = D / 2;
  for (int i = 0; i < half; ++i) {
    const double f = pow(theta, -(2.0 * i) / (double)D);
    const double a = x[i], b = x[i + half], ang = pos * f;
    const double cs = cos(ang), sn = sin(ang);
    y[i] = a * cs - b * sn;
    y[i + half] = a * sn + b * cs;
  }
}

/* out = softmax(q' K'^T / sqrt(D)) V over the first T tokens of one kv head's cache,
 * for one query vector q (fp16 [D], rotated at position q_pos): the attention step of
 * the decode loop over the dequantized cache ([TQ] section 4.2: the quantized cache is
 * dequantized before it is used; [KVC3] "Pre-RoPE Key Quantization": keys are rotated
 * at their own position when read).  Sums run in ascending t. */
static int orc_attend(const orc_cfg *c, const orc_head *hd, const uint16_t *q, int64_t q_pos,
                      int64_t T, double *out) {
  const int D = c->head_dim;
  if (T <= 0 || T > hd->length) return -1;
  double *qx = (double *)malloc(sizeof(double) * D * 4);
  float *row = (float *)malloc(sizeof(float) * D);
  double *s = (double *)malloc(sizeof(double) * (size_t)T);
  if (!qx || !row || !s) { free(qx); free(row); free(s); return -1; }
  double *qr = qx + D, *kx = qx + 2 * D, *kr = qx + 3 * D;
  for (int i = 0; i < D; ++i) qx[i] = (double)orc_h2f(q[i]);
  orc_rope(qx, qr, D, (double)q_pos, (double)c->rope_theta);
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  double m = -INFINITY;
  for (int64_t t = 0; t < T; ++t) {
    orc_dequant_row(c, hd, 0, t, row);
    for (int i = 0; i < D; ++i) kx[i] = (double)row[i];
    orc_rope(kx, kr, D, (double)t, (double)c->rope_theta);
    double acc = 0.0;
    for (int i = 0; i < D; ++i) acc += qr[i] * kr[i];
    s[t] = acc * inv_sqrt_d;
    if (s[t] > m) m = s[t];
  }
  double l = 0.0;
  for (int i = 0; i < D; ++i) out[i] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const double w = exp(s[t] - m);
    l += w;
    orc_dequant_row(c, hd, 1, t, row);
    for (int i = 0; i < D; ++i) out[i] += w * (double)row[i];
  }
  for (int i = 0; i < D; ++i) out[i] /= l;
  free(qx);
  free(row);
  free(s);
  return 0;
}

/* Single-query decode: the query attends to every token the cache holds. */
int orc_decode_head(const orc_cfg *c, const orc_head *hd, const uint16_t *q, int64_t q_pos,
                    double *out) {
  return orc_attend(c, hd, q, q_pos, hd->length, out);
}

/* A chunk of nq consecutive query tokens (a prefill chunk, or the draft tokens of a
 * speculative-verification step; [UQ] section 5.1 counts first-token latency among
 * the costs to evaluate): query j (fp16 [D] at q + j*D) sits at position q_pos + j
 * and attends causally, to the cache tokens t <= q_pos + j, i.e. to the first
 * min(q_pos + j + 1, length) of them.  out is [nq][D]. */
int orc_chunk_head(const orc_cfg *c, const orc_head *hd, const uint16_t *q, int32_t nq,
                   int64_t q_pos, double *out) {
  if (nq <= 0 || q_pos < 0) return -1;
  for (int32_t j = 0; j < nq; ++j) {
    int64_t nvis = q_pos + j + 1;
    if (nvis > hd->length) nvis = hd->length;
    if (orc_attend(c, hd, q + (int64_t)j * c->head_dim, q_pos + j, nvis, out + (int64_t)j * c->head_dim))
      return -1;
  }
  return 0;
}

/* Several independent (query, kv head) pairs; results do not depend on the
 * number of threads. */
int orc_decode_many(const orc_cfg *c, int64_t n, const orc_head *const *hds,
                    const uint16_t *qs, const int64_t *q_pos, double *outs) {
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int64_t i = 0; i < n; ++i)
    err |= orc_decode_head(c, hds[i], qs + i * c->head_dim, q_pos[i], outs + i * c->head_dim) != 0;
  return err ? -1 : 0;
}

/* Several independent (query chunk, kv head) pairs: chunk i is nq queries at
 * qs + i*nq*D, positions q_pos[i] .. q_pos[i] + nq - 1, output outs + i*nq*D. */
int orc_chunk_many(const orc_cfg *c, int64_t n, const orc_head *const *hds, const uint16_t *qs,
                   int32_t nq, const int64_t *q_pos, double *outs) {
  int err = 0;
  const int64_t stride = (int64_t)nq * c->head_dim;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int64_t i = 0; i < n; ++i)
    err |= orc_chunk_head(c, hds[i], qs + i * stride, nq, q_pos[i], outs + i * stride) != 0;
  return err ? -1 : 0;
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
