/* Runs the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer on small
 * caches whose buffers are allocated to their exact layout sizes, so that any read or
 * write past a buffer, any signed overflow or any misaligned access in the oracle is
 * reported.  Covers uniform and codebook keys, 2/3/4-bit codes, head sizes 64 and 128,
 * clipping, outliers, keys kept in fp16, codebook values, ragged tails, dequantization
 * and decode.  Exit
 * status 0 = clean. */
#include "../../oracle/oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double unif(void) { /* xorshift64*, uniform in [0, 1) */
  rng_state ^= rng_state >> 12; rng_state ^= rng_state << 25; rng_state ^= rng_state >> 27;
  return (double)((rng_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static uint16_t f16_of(double x) { return orc_f2h_rn((float)x); }

static void *xalloc(int64_t n) { return n > 0 ? malloc((size_t)n) : NULL; }

static int run(orc_cfg c, int64_t T) {
  int64_t lay[18];
  orc_layout(&c, lay);
  const int D = c.head_dim;
  orc_head h;
  memset(&h, 0, sizeof h);
  /* one (b, h) slice of each buffer: the layout sizes divided by batch * kv_heads */
  const int64_t bh = (int64_t)c.batch * c.kv_heads;
  h.k_codes = xalloc(lay[0] / bh); h.k_scale = xalloc(lay[1] / bh); h.k_zero = xalloc(lay[2] / bh);
  uint16_t *lut = xalloc(lay[3] / c.kv_heads);
  if (lut) {
    const int nl = 1 << c.k_bits;
    for (int d = 0; d < D; ++d)
      for (int k = 0; k < nl; ++k) lut[d * nl + k] = f16_of(-2.0 + 4.0 * (k + 0.5) / nl);
  }
  h.k_lut = lut;
  h.k_tail = xalloc(lay[4] / bh); h.v_codes = xalloc(lay[5] / bh); h.v_scale = xalloc(lay[6] / bh);
  h.v_zero = xalloc(lay[7] / bh); h.v_tail = xalloc(lay[8] / bh);
  h.k_rowptr = xalloc(lay[9] / bh); h.k_col = xalloc(lay[10] / bh); h.k_val = xalloc(lay[11] / bh);
  h.v_rowptr = xalloc(lay[12] / bh); h.v_col = xalloc(lay[13] / bh); h.v_val = xalloc(lay[14] / bh);
  h.k_keep_idx = xalloc(lay[15] / bh); h.k_keep_val = xalloc(lay[16] / bh);
  uint16_t *vlut = xalloc(lay[17] / c.kv_heads);
  if (vlut) {
    const int nl = 1 << c.v_bits;
    for (int d = 0; d < D; ++d)
      for (int k = 0; k < nl; ++k) vlut[d * nl + k] = f16_of(-1.5 + 3.0 * (k + 0.5) / nl);
  }
  h.v_lut = vlut;
  uint16_t *k = malloc((size_t)(T * D) * 2), *v = malloc((size_t)(T * D) * 2);
  for (int64_t i = 0; i < T * D; ++i) {
    const double heavy = unif() < 0.02 ? 40.0 : 1.0;
    k[i] = f16_of((unif() * 2.0 - 1.0) * 3.0 * heavy);
    v[i] = f16_of((unif() * 2.0 - 1.0) * 2.0 * heavy);
  }
  int err = orc_build_head(&c, &h, k, v, T);
  float *deq = malloc((size_t)(T * D) * sizeof(float));
  for (int which = 0; which < 2 && !err; ++which) err |= orc_dequantize_head(&c, &h, which, 0, T, deq);
  uint16_t q[256];
  for (int d = 0; d < D; ++d) q[d] = f16_of(unif() * 2.0 - 1.0);
  double out[256];
  const int64_t pos[3] = {T - 1, T + 1000, 3};
  for (int i = 0; i < 3 && !err; ++i) err |= orc_decode_head(&c, &h, q, pos[i], out);
  /* a chunk of 5 queries in buffers of exactly 5 rows, the last rows past the end */
  uint16_t *qc = malloc((size_t)(5 * D) * 2);
  double *oc = malloc((size_t)(5 * D) * sizeof(double));
  for (int64_t i = 0; i < 5 * D; ++i) qc[i] = f16_of(unif() * 2.0 - 1.0);
  if (!err) err |= orc_chunk_head(&c, &h, qc, 5, T - 3, oc);
  if (!err) err |= orc_chunk_head(&c, &h, qc, 5, 0, oc);
  free(qc); free(oc);
  const int64_t nblk = T / c.k_block;
  if (nblk > 0) (void)orc_clip_threshold(k, (int64_t)c.k_block * D, 0.99f);
  free(deq); free(k); free(v); free(lut); free(vlut);
  free(h.k_codes); free(h.k_scale); free(h.k_zero); free(h.k_tail); free(h.v_codes); free(h.v_scale);
  free(h.v_zero); free(h.v_tail); free(h.k_rowptr); free(h.k_col); free(h.k_val); free(h.v_rowptr);
  free(h.v_col); free(h.v_val); free(h.k_keep_idx); free(h.k_keep_val);
  return err;
}

int main(void) {
  /* batch, q_heads, kv_heads, D, capacity, k_bits, k_mode, k_block, v_bits, v_group, clip, pct, theta,
   * keep, v_mode */
  const orc_cfg cfgs[] = {
      {1, 4, 4, 64, 320, 4, 0, 64, 4, 64, 0.0f, 0, 10000.0f},
      {1, 2, 2, 128, 768, 4, 0, 128, 4, 128, 0.99f, 1, 10000.0f},
      {1, 8, 2, 128, 640, 4, 0, 128, 2, 64, 0.0f, 1, 10000.0f},
      {1, 2, 2, 128, 768, 3, 1, 128, 2, 64, 0.0f, 0, 10000.0f},
      {1, 2, 2, 64, 384, 2, 1, 64, 4, 32, 0.9f, 2, 10000.0f},
      {1, 2, 2, 128, 384, 3, 0, 128, 4, 32, 0.0f, 3, 500000.0f},
      {1, 4, 4, 64, 256, 2, 0, 64, 2, 16, 0.5f, 0, 10000.0f},
      {1, 2, 2, 128, 512, 4, 0, 128, 4, 128, 0.0f, 0, 10000.0f, 12},
      {1, 8, 2, 64, 320, 3, 0, 64, 2, 32, 0.0f, 0, 10000.0f, 25},
      {1, 2, 2, 128, 512, 4, 0, 128, 4, 128, 0.0f, 0, 10000.0f, 0, 1},
      {1, 8, 2, 64, 320, 3, 1, 64, 2, 32, 0.0f, 0, 10000.0f, 0, 1},
  };
  const int64_t lens[] = {293, 697, 589, 643, 333, 300, 200, 450, 301, 400, 250};
  int err = 0;
  for (size_t i = 0; i < sizeof cfgs / sizeof cfgs[0]; ++i) {
    const int e = run(cfgs[i], lens[i]);
    printf("config %zu: %s\n", i, e ? "error" : "ok");
    err |= e;
  }
  return err ? 1 : 0;
}
