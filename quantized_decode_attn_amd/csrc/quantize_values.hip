// quantize_values.hip -- the value-block kernels (see quantize_block.h for the steps).
#include "quantize_block.h"

namespace kvq {
namespace {

// Codebook values (v_mode 1): the code of x is its nearest entry among the channel's
// sorted fp16 centroids, decided at the fp32 midpoints (C[k] + C[k+1]) / 2 with ties to
// the lower code ([KVC3] "Non-Uniform KV Cache Quantization", which names the Value
// cache first; a log-spaced codebook is the log quantization of [TQ] section 3.3).
// Elementwise: no statistics, outliers or clipping.  The code is the number of
// midpoints below x, found by a binary search over the channel's midpoints in LDS
// (they never decrease, so the search and the count agree; NaN compares false and gets
// code 0).  A thread takes one token group (32 / VB tokens) of 8 channels: a 16-byte
// load per token row (from the tail or from the new rows), 8 words out (one channel,
// the group's tokens, as the uniform kernel stores them).  The midpoints are stored
// index-major, [k][D], so that a wave's lookups spread over the banks by channel.
template <int D, int BK, int VB>
__global__ __launch_bounds__(qb::kThreads) void quantize_values_lut_kernel(kvq_cache c, const uint16_t* __restrict__ v_new,
                                                                           int64_t old_len_arg, int64_t n_new,
                                                                           int64_t n_first, const int64_t* __restrict__ n_seq) {
  constexpr int NL = 1 << VB, L = NL - 1;
  constexpr int TPW = 32 / VB;
  constexpr int NTASK = (BK / TPW) * (D / 8);  // (token group, channel octet) pairs
  __shared__ float mid[L * D];
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t old_len = c.seq_lens ? seq_len_of(c, b) : old_len_arg;
  const int64_t n_b = n_seq ? min(max(n_seq[b], (int64_t)0), n_new) : n_new;
  const int64_t n = (c.seq_lens ? old_len / BK : n_first) + blockIdx.x;
  if (n >= (old_len + n_b) / BK || n >= c.cfg.capacity / BK) return;
  const int64_t g = slot_of(c, b, h, n);
  const int64_t bh = (int64_t)b * c.cfg.kv_heads + h;
  const uint16_t* lut = c.v_lut + (int64_t)h * D * NL;
  for (int k = threadIdx.x; k < D * L; k += qb::kThreads) {
    const int ch = k / L, e = k % L;
    mid[e * D + ch] = (h2f(lut[ch * NL + e]) + h2f(lut[ch * NL + e + 1])) * 0.5f;
  }
  __syncthreads();
  const int64_t t0 = n * BK, tail0 = (old_len / BK) * BK;
  uint32_t* words = static_cast<uint32_t*>(c.v_codes) + g * (BK / TPW) * D;
  for (int task = threadIdx.x; task < NTASK; task += qb::kThreads) {
    const int tg = task / (D / 8), c0 = 8 * (task % (D / 8));
    uint32_t wd[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int64_t t = t0 + tg * TPW + u;
      const uint16_t* row = t < old_len ? c.v_tail + (bh * BK + (t - tail0)) * D
                                        : v_new + (bh * n_new + (t - old_len)) * D;
      const uint4 x4 = *reinterpret_cast<const uint4*>(row + c0);
      const uint32_t xw[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = h2f((uint16_t)(xw[e >> 1] >> (16 * (e & 1))));
        const float* m = mid + c0 + e;
        uint32_t code = 0u;
#pragma unroll
        for (int step = NL / 2; step >= 1; step >>= 1)
          code += x > m[(code + step - 1) * D] ? (uint32_t)step : 0u;
        wd[e] |= code << (u * VB);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) words[tg * D + c0 + e] = wd[e];
  }
}

template <int D, int BK, int VB>
hipError_t launch_v_lut(const kvq_cache& c, const uint16_t* v_new, int64_t old_len, int64_t n_new,
                        int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  dim3 grid((unsigned)nblocks, (unsigned)c.cfg.kv_heads, (unsigned)c.cfg.batch);
  hipLaunchKernelGGL((quantize_values_lut_kernel<D, BK, VB>), grid, dim3(qb::kThreads), 0, s, c, v_new, old_len,
                     n_new, n_first, n_seq);
  return hipGetLastError();
}

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
  if (c.cfg.v_mode == 1) return launch_v_lut<D, BK, VB>(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
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
