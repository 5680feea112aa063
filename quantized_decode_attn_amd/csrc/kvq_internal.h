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

// Key vectors kept in fp16 per quantized block (keep_pct > 0).
__host__ __device__ inline int keep_count(const kvq_config& c) {
  return c.keep_pct > 0 ? (c.keep_pct * c.k_block + 99) / 100 : 0;
}

hipError_t launch_rope_init(const kvq_cache& c, hipStream_t s);

// Quantize the complete blocks [n_first, n_first + nblocks) of every (b, kv-head).
// Tokens below `old_len` come from the tails, the others from the new input
// (row t - old_len of `k_new`/`v_new`, each [B][Hkv][n_new][D]).  In a paged cache
// every sequence uses its own length from the device array instead of old_len and
// n_first, and nblocks is the most blocks any sequence completes.
// n_seq (device, per sequence; caches with per-sequence lengths only): each sequence's
// count of new tokens, n_new then being the input's rows per sequence.
hipError_t launch_quantize(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                           int64_t old_len, int64_t n_new, int64_t n_first, int64_t nblocks,
                           hipStream_t s, const int64_t* n_seq = nullptr);

// The parts of launch_quantize: one kernel per tensor (uniform or codebook keys).
hipError_t launch_quantize_keys_uniform(const kvq_cache& c, const uint16_t* k_new, int64_t old_len,
                                        int64_t n_new, int64_t n_first, int64_t nblocks, const int64_t* n_seq,
                                        hipStream_t s);
hipError_t launch_quantize_keys_lut(const kvq_cache& c, const uint16_t* k_new, int64_t old_len, int64_t n_new,
                                    int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s);
hipError_t launch_quantize_values(const kvq_cache& c, const uint16_t* v_new, int64_t old_len, int64_t n_new,
                                  int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s);
// FP8 cache (k_mode 2 with v_mode 2): both tensors of each completed block in one kernel.
hipError_t launch_quantize_fp8(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new, int64_t old_len,
                               int64_t n_new, int64_t n_first, int64_t nblocks, const int64_t* n_seq,
                               hipStream_t s);

// Copy new rows [src0, n_new) into tail slots [dst0, ...) (a paged cache: per
// sequence, from its own length).
hipError_t launch_tail_copy(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                            int64_t n_new, int64_t src0, int64_t dst0, hipStream_t s,
                            const int64_t* n_seq = nullptr);
// A paged cache's device lengths advance by n, or by n_seq[b] (stream-ordered after the
// append).
hipError_t launch_seq_lens_add(const kvq_cache& c, int64_t n, hipStream_t s, const int64_t* n_seq = nullptr);
// ... or are set to n (the cache's initialisation).
hipError_t launch_seq_lens_set(const kvq_cache& c, int64_t n, hipStream_t s);

// q_pos < 0 (caches with per-sequence lengths): every sequence at its own newest token.
hipError_t launch_decode(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* out,
                         float* ws, int splits, hipStream_t s);

// Rows of the split kernels: query vectors (query head g of a kv head, query j of a
// chunk of nq; q and out are [B][Hq][nq][D]) with their rotation position q_pos + j
// and the cache tokens they see.
struct RowSpec {
  int64_t q_pos;  // position of query 0
  int nq;         // queries per query head
  int causal;     // 1: query j sees the tokens t <= q_pos + j; 0: the whole cache
  int rpi;        // rows per work item (set by the launcher of the generic kernel)
  int nsets;      // row sets per kv head (idem)
};

__host__ __device__ inline int64_t row_visible(const RowSpec& rs, int j, int64_t length) {
  if (!rs.causal) return length;
  const int64_t n = rs.q_pos + j + 1;
  return n < length ? n : length;
}

// Fused decode step over a cache whose length already counts the new token; the new
// token's keys and values [B][Hkv][D] stand at tail slot jnew (read from the input,
// written to the tail), or jnew < 0 when the token completed a block that is already
// quantized.  splits == 0: one launch, one workgroup per (b, kv-head) whose waves take
// the splits, merged in LDS (hipErrorNotSupported when the rows of a kv head do not fit
// one workgroup; ws unused).  splits > 0: the decode split kernel with that many splits
// and the finish kernel, partials in ws.
hipError_t launch_decode_step(const kvq_cache& c, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                              int jnew, float* out, float* ws, int splits, hipStream_t s);
// Whether a decode step on a short cache should take the one-launch kernel: every query
// head of a kv head fits its workgroup, and no tuned split kernel covers the
// configuration (host only).
bool decode_step_prefers_one_launch(const kvq_cache& c);

// Causal attention of a chunk of nq queries (the generic split kernel, or the
// matrix-core kernel where it applies), partials merged by the finish kernel.
hipError_t launch_chunk(const kvq_cache& c, const uint16_t* q, int nq, int64_t q_pos, float* out,
                        float* ws, int splits, hipStream_t s);

// The matrix-core chunk kernel; hipErrorNotSupported for configurations it does not cover.
hipError_t launch_chunk_mfma(const kvq_cache& c, const uint16_t* q, RowSpec rs, float* ws, int S,
                             hipStream_t s, int cus);

hipError_t launch_dequantize(const kvq_cache& c, int which, int64_t t0, int64_t t1, float* out,
                             hipStream_t s);

}  // namespace kvq
