// quantize_keys.hip -- the uniform key-block kernels (see quantize_block.h for the steps).
#include "quantize_block.h"

#ifndef KVQ_KEYS_LUT
#define KVQ_KEYS_LUT false
#define KVQ_KEYS_ENTRY launch_quantize_keys_uniform
#endif

namespace kvq {
namespace {

template <int D, int BK, int LUTB, bool OUTL, bool CLIP>
hipError_t launch_k(const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                    int64_t n_first, int64_t nblocks, hipStream_t s) {
  dim3 grid((unsigned)nblocks, (unsigned)c.cfg.kv_heads, (unsigned)c.cfg.batch);
  hipLaunchKernelGGL((qb::quantize_keys_kernel<D, BK, LUTB, OUTL, CLIP>), grid, dim3(qb::kThreads), 0, s, c, k_new,
                     old_len, n_new, n_first);
  return hipGetLastError();
}

template <int D, int BK, int LUTB>
hipError_t dispatch_k(const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                      int64_t n_first, int64_t nblocks, hipStream_t s) {
  const bool outl = kvq::host_kout(c.cfg) > 0, clip = c.cfg.clip_quantile > 0.0f;
  if (outl && clip) return launch_k<D, BK, LUTB, true, true>(c, k_new, old_len, n_new, n_first, nblocks, s);
  if (outl) return launch_k<D, BK, LUTB, true, false>(c, k_new, old_len, n_new, n_first, nblocks, s);
  if (clip) return launch_k<D, BK, LUTB, false, true>(c, k_new, old_len, n_new, n_first, nblocks, s);
  return launch_k<D, BK, LUTB, false, false>(c, k_new, old_len, n_new, n_first, nblocks, s);
}

template <int LUTB>
hipError_t dispatch_bk(int D, int Bk, const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                       int64_t n_first, int64_t nblocks, hipStream_t s) {
  if (D == 128 && Bk == 128) return dispatch_k<128, 128, LUTB>(c, k_new, old_len, n_new, n_first, nblocks, s);
  if (D == 128 && Bk == 64) return dispatch_k<128, 64, LUTB>(c, k_new, old_len, n_new, n_first, nblocks, s);
  if (D == 64 && Bk == 128) return dispatch_k<64, 128, LUTB>(c, k_new, old_len, n_new, n_first, nblocks, s);
  if (D == 64 && Bk == 64) return dispatch_k<64, 64, LUTB>(c, k_new, old_len, n_new, n_first, nblocks, s);
  return hipErrorInvalidValue;
}

}  // namespace

// Keys with a per-channel codebook (k_mode 1) or uniform keys, by the file's LUT flag.
hipError_t KVQ_KEYS_ENTRY(const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                          int64_t n_first, int64_t nblocks, hipStream_t s) {
  const int D = c.cfg.head_dim, Bk = c.cfg.k_block;
  if constexpr (KVQ_KEYS_LUT) {
    const int kb = c.cfg.k_bits;
    if (kb == 2) return dispatch_bk<2>(D, Bk, c, k_new, old_len, n_new, n_first, nblocks, s);
    if (kb == 3) return dispatch_bk<3>(D, Bk, c, k_new, old_len, n_new, n_first, nblocks, s);
    if (kb == 4) return dispatch_bk<4>(D, Bk, c, k_new, old_len, n_new, n_first, nblocks, s);
    return hipErrorInvalidValue;
  }
  return dispatch_bk<0>(D, Bk, c, k_new, old_len, n_new, n_first, nblocks, s);
}

}  // namespace kvq
