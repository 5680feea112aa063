// kvq_internal.h -- launchers shared between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// Outliers per token vector: ceil(pct * head_dim / 100).
inline int host_kout(const kvq_config& c) {
  return c.outlier_pct > 0 ? (c.outlier_pct * c.head_dim + 99) / 100 : 0;
}

hipError_t launch_rope_init(const kvq_cache& c, hipStream_t s);

// Quantize the complete blocks [n_first, n_first + nblocks) of every (b, kv-head).
// Tokens below `old_len` come from the tails, the others from the new input
// (row t - old_len of `k_new`/`v_new`, each [B][Hkv][n_new][D]).
hipError_t launch_quantize(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                           int64_t old_len, int64_t n_new, int64_t n_first, int64_t nblocks,
                           hipStream_t s);

// The parts of launch_quantize: one kernel per tensor (uniform or codebook keys).
hipError_t launch_quantize_keys_uniform(const kvq_cache& c, const uint16_t* k_new, int64_t old_len,
                                        int64_t n_new, int64_t n_first, int64_t nblocks, hipStream_t s);
hipError_t launch_quantize_keys_lut(const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                                    int64_t n_first, int64_t nblocks, hipStream_t s);
hipError_t launch_quantize_values(const kvq_cache& c, const uint16_t* v_new, int64_t old_len, int64_t n_new,
                                  int64_t n_first, int64_t nblocks, hipStream_t s);

// Copy new rows [src0, n_new) into tail slots [dst0, ...).
hipError_t launch_tail_copy(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                            int64_t n_new, int64_t src0, int64_t dst0, hipStream_t s);

hipError_t launch_decode(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* out,
                         float* ws, int splits, hipStream_t s);

hipError_t launch_dequantize(const kvq_cache& c, int which, int64_t t0, int64_t t1, float* out,
                             hipStream_t s);

}  // namespace kvq
