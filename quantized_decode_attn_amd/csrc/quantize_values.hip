// quantize_values.hip -- the value-block kernels (see quantize_block.h for the steps).
#include "quantize_block.h"

namespace kvq {
namespace {

template <int D, int BK, int VB, int KO, bool CLIP>
hipError_t launch_v(const kvq_cache& c, const uint16_t* v_new, int64_t old_len, int64_t n_new,
                    int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  dim3 grid((unsigned)nblocks, (unsigned)c.cfg.kv_heads, (unsigned)c.cfg.batch);
  hipLaunchKernelGGL((qb::quantize_values_kernel<D, BK, VB, KO, CLIP>), grid, dim3(qb::kThreads), 0, s, c,
                     v_new, old_len, n_new, n_first, n_seq);
  return hipGetLastError();
}

template <int D, int BK, int VB>
hipError_t dispatch_v(const kvq_cache& c, const uint16_t* v_new, int64_t old_len, int64_t n_new,
                      int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  // outliers per vector: none, exactly two (the 1% of 128 channels), or any other count
  // (1..4, read at run time)
  const int ko = kvq::host_kout(c.cfg);
  const bool clip = c.cfg.clip_quantile > 0.0f;
#define KVQ_V(KO)                                                                                  \
  return clip ? launch_v<D, BK, VB, KO, true>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s)       \
              : launch_v<D, BK, VB, KO, false>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (ko == 0) { KVQ_V(0) }
  if (ko == 2) { KVQ_V(2) }
  KVQ_V(-1)
#undef KVQ_V
}

template <int D, int BK>
hipError_t dispatch_vb(const kvq_cache& c, const uint16_t* v_new, int64_t old_len, int64_t n_new,
                       int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  if (c.cfg.v_bits == 4) return dispatch_v<D, BK, 4>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (c.cfg.v_bits == 2) return dispatch_v<D, BK, 2>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize_values(const kvq_cache& c, const uint16_t* v_new, int64_t old_len, int64_t n_new,
                                  int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  const int D = c.cfg.head_dim, Bk = c.cfg.k_block;
  if (D == 128 && Bk == 128) return dispatch_vb<128, 128>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 128 && Bk == 64) return dispatch_vb<128, 64>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 64 && Bk == 128) return dispatch_vb<64, 128>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 64 && Bk == 64) return dispatch_vb<64, 64>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
