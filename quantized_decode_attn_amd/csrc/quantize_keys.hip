// quantize_keys.hip -- the uniform key-block kernels (see quantize_block.h for the steps).
#include "quantize_block.h"

#ifndef KVQ_KEYS_LUT
#define KVQ_KEYS_LUT false
#define KVQ_KEYS_ENTRY launch_quantize_keys_uniform
#endif

namespace kvq {
namespace {

template <int D, int BK, int LUTB, int KO, bool CLIP, bool RET = false>
hipError_t launch_k(const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                    int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  dim3 grid((unsigned)nblocks, (unsigned)c.cfg.kv_heads, (unsigned)c.cfg.batch);
  hipLaunchKernelGGL((qb::quantize_keys_kernel<D, BK, LUTB, KO, CLIP, RET>), grid, dim3(qb::kThreads), 0, s, c, k_new,
                     old_len, n_new, n_first, n_seq);
  return hipGetLastError();
}

template <int D, int BK, int LUTB>
hipError_t dispatch_k(const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                      int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  // outliers per vector: none, exactly two (the 1% of 128 channels), or any other count
  // (1..4, read at run time); uniform keys only get the two-outlier specialisation
  const int ko = kvq::host_kout(c.cfg);
  const bool clip = c.cfg.clip_quantile > 0.0f;
  if constexpr (LUTB == 0)  // keys kept in fp16 (no outliers, no clipping)
    if (c.cfg.keep_pct > 0) return launch_k<D, BK, 0, 0, false, true>(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
#define KVQ_K(KO)                                                                                  \
  return clip ? launch_k<D, BK, LUTB, KO, true>(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s)     \
              : launch_k<D, BK, LUTB, KO, false>(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (ko == 0) { KVQ_K(0) }
  if constexpr (LUTB == 0)
    if (ko == 2) { KVQ_K(2) }
  KVQ_K(-1)
#undef KVQ_K
}

template <int LUTB>
hipError_t dispatch_bk(int D, int Bk, const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                       int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  if (D == 128 && Bk == 128) return dispatch_k<128, 128, LUTB>(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 128 && Bk == 64) return dispatch_k<128, 64, LUTB>(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 64 && Bk == 128) return dispatch_k<64, 128, LUTB>(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 64 && Bk == 64) return dispatch_k<64, 64, LUTB>(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
  return hipErrorInvalidValue;
}

}  // namespace

// Keys with a per-channel codebook (k_mode 1) or uniform keys, by the file's LUT flag.
hipError_t KVQ_KEYS_ENTRY(const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                          int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  const int D = c.cfg.head_dim, Bk = c.cfg.k_block;
  if constexpr (KVQ_KEYS_LUT) {
    const int kb = c.cfg.k_bits;
    if (kb == 2) return dispatch_bk<2>(D, Bk, c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
    if (kb == 3) return dispatch_bk<3>(D, Bk, c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
    if (kb == 4) return dispatch_bk<4>(D, Bk, c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
    return hipErrorInvalidValue;
  }
  return dispatch_bk<0>(D, Bk, c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
}

}  // namespace kvq
