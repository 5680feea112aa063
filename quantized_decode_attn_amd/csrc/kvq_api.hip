// kvq_api.hip -- the C ABI: argument checking, buffer sizes, launch sequencing.
// Nothing here allocates device memory; every launch goes on the caller's stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

kvq_status check_cfg(const kvq_config* c) {
  if (!c) return KVQ_EINVAL;
  if (c->batch <= 0 || c->q_heads <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 || c->capacity <= 0)
    return KVQ_EINVAL;
  if (c->head_dim % 2 || c->q_heads % c->kv_heads) return KVQ_EINVAL;
  if (c->k_bits < 1 || c->k_bits > 8 || c->v_bits < 1 || c->v_bits > 8) return KVQ_EINVAL;
  if (c->k_mode < 0 || c->k_mode > 2) return KVQ_EINVAL;
  if (c->k_block <= 0 || c->capacity % c->k_block) return KVQ_EINVAL;
  if (c->v_group <= 0 || c->head_dim % c->v_group) return KVQ_EINVAL;
  if (!(c->clip_quantile >= 0.0f && c->clip_quantile < 1.0f)) return KVQ_EINVAL;
  if (c->outlier_pct < 0 || c->outlier_pct > 100) return KVQ_EINVAL;
  if (!(c->rope_theta > 1.0f) || !isfinite(c->rope_theta)) return KVQ_EINVAL;
  if (c->keep_pct < 0 || c->keep_pct > 100) return KVQ_EINVAL;
  if (c->v_mode < 0 || c->v_mode > 2) return KVQ_EINVAL;
  // FP8: keys and values together, one byte per element
  if ((c->k_mode == 2) != (c->v_mode == 2)) return KVQ_EINVAL;
  if (c->k_mode == 2 && (c->k_bits != 8 || c->v_bits != 8)) return KVQ_EINVAL;
  // what the kernels are built for
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_EUNSUPPORTED;
  if (c->k_mode != 2 && (c->k_bits < 2 || c->k_bits > 4)) return KVQ_EUNSUPPORTED;
  if (c->v_mode != 2 && c->v_bits != 2 && c->v_bits != 4) return KVQ_EUNSUPPORTED;
  if (c->v_group != 16 && c->v_group != 32 && c->v_group != 64 && c->v_group != 128)
    return KVQ_EUNSUPPORTED;
  if (c->k_block != 64 && c->k_block != 128) return KVQ_EUNSUPPORTED;
  if (c->q_heads / c->kv_heads > 8) return KVQ_EUNSUPPORTED;
  if (kvq::host_kout(*c) > 4) return KVQ_EUNSUPPORTED;
  // kept fp16 keys: up to 16 per block, with uniform keys, no outliers, no clipping
  if (kvq::keep_count(*c) > 16) return KVQ_EUNSUPPORTED;
  if (c->keep_pct > 0 && (c->k_mode != 0 || c->outlier_pct > 0 || c->clip_quantile > 0.0f))
    return KVQ_EUNSUPPORTED;
  // codebook or FP8 values: no outliers, no clipping (both belong to the uniform range)
  if (c->v_mode != 0 && (c->outlier_pct > 0 || c->clip_quantile > 0.0f)) return KVQ_EUNSUPPORTED;
  if (c->k_mode == 2 && c->keep_pct > 0) return KVQ_EUNSUPPORTED;
  return KVQ_OK;
}

kvq_status check_cache(const kvq_cache* cache) {
  if (!cache) return KVQ_EINVAL;
  kvq_status st = check_cfg(&cache->cfg);
  if (st != KVQ_OK) return st;
  const kvq_config& c = cache->cfg;
  if (!cache->k_codes || !cache->k_tail || !cache->v_codes || !cache->v_tail || !cache->rope)
    return KVQ_EINVAL;
  if (c.v_mode == 0 && (!cache->v_scale || !cache->v_zero)) return KVQ_EINVAL;
  if (c.v_mode == 1 && !cache->v_lut) return KVQ_EINVAL;
  if (c.k_mode == 0 && (!cache->k_scale || !cache->k_zero)) return KVQ_EINVAL;
  if (c.k_mode == 1 && !cache->k_lut) return KVQ_EINVAL;
  if (kvq::host_kout(c) > 0 && (!cache->k_rowptr || !cache->k_col || !cache->k_val ||
                                !cache->v_rowptr || !cache->v_col || !cache->v_val))
    return KVQ_EINVAL;
  if (kvq::keep_count(c) > 0 && (!cache->k_keep_idx || !cache->k_keep_val)) return KVQ_EINVAL;
  if (cache->length < 0 || cache->length > c.capacity) return KVQ_EINVAL;
  // per-sequence lengths (both copies or neither); a block table needs them
  if (!cache->seq_lens != !cache->seq_lens_host) return KVQ_EINVAL;
  if (cache->block_table && !cache->seq_lens) return KVQ_EINVAL;
  if (cache->block_table && (cache->num_blocks < 1 || (int64_t)cache->num_blocks * c.kv_heads >= ((int64_t)1 << 31)))
    return KVQ_EINVAL;
  if (cache->seq_lens_host)
    for (int b = 0; b < c.batch; ++b)
      if (cache->seq_lens_host[b] < 0 || cache->seq_lens_host[b] > c.capacity) return KVQ_EINVAL;
  return KVQ_OK;
}

bool per_sequence(const kvq_cache* cache) { return cache->seq_lens != nullptr; }

// A decode's query position: a cache with per-sequence lengths takes -1 (every sequence
// at its own newest token; each must hold one), a dense one a position in [0, 2^40].
kvq_status check_decode_pos(const kvq_cache* cache, int64_t q_pos) {
  if (per_sequence(cache)) {
    if (q_pos != -1) return KVQ_EINVAL;
    for (int b = 0; b < cache->cfg.batch; ++b)
      if (cache->seq_lens_host[b] < 1) return KVQ_EINVAL;
    return KVQ_OK;
  }
  if (q_pos < 0 || q_pos > ((int64_t)1 << 40) || cache->length == 0) return KVQ_EINVAL;
  return KVQ_OK;
}

kvq_status from_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_EHIP; }

// The append of a cache with per-sequence lengths: sequence b takes count(b) =
// n_host ? n_host[b] : n_rows tokens, the first of its n_rows input rows.  The kernels
// read the device lengths (and n_dev), the host copies size the launches; every check
// comes before the first launch, and the host lengths advance only when every launch
// was enqueued.
kvq_status append_per_sequence(kvq_cache* cache, const uint16_t* kn, const uint16_t* vn, int64_t n_rows,
                               const int64_t* n_host, const int64_t* n_dev, hipStream_t s) {
  const kvq_config& c = cache->cfg;
  int64_t most_blocks = 0;
  bool tail = false;
  for (int b = 0; b < c.batch; ++b) {
    const int64_t L0 = cache->seq_lens_host[b], L1 = L0 + (n_host ? n_host[b] : n_rows);
    if (L1 > c.capacity) return KVQ_ECAPACITY;
    const int64_t nb = L1 / c.k_block - L0 / c.k_block;
    most_blocks = nb > most_blocks ? nb : most_blocks;
    tail = tail || (L1 % c.k_block != 0 && L1 != L0);
  }
  kvq_status st = KVQ_OK;
  if (most_blocks > 0) {
    st = from_hip(kvq::launch_quantize(*cache, kn, vn, 0, n_rows, 0, most_blocks, s, n_dev));
    if (st != KVQ_OK) return st;
  }
  if (tail) {
    st = from_hip(kvq::launch_tail_copy(*cache, kn, vn, n_rows, 0, 0, s, n_dev));
    if (st != KVQ_OK) return st;
  }
  st = from_hip(kvq::launch_seq_lens_add(*cache, n_rows, s, n_dev));
  if (st != KVQ_OK) return st;
  for (int b = 0; b < c.batch; ++b) cache->seq_lens_host[b] += n_host ? n_host[b] : n_rows;
  return KVQ_OK;
}

// Device-side split partials of kvq_decode_attention_noalloc: one array per GPU the
// library runs on (the code object's copy on that device), held until the process ends.
constexpr size_t kNoallocScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current GPU's `scratch`, looked up once per device with
// that device current (the host-side name is only a stand-in for it).
kvq_status scratch_of_current_device(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return KVQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return KVQ_OK;
}

int auto_splits(const kvq_config& c) {
  // About one (b, kv-head, split) work item per resident wave of an MI355X (256 CUs x
  // 8 waves), without splitting a sequence below one block per split.
  const int64_t units = (int64_t)c.batch * c.kv_heads;
  int64_t s = (2048 + units - 1) / units;
  const int64_t nblk = c.capacity / c.k_block;
  if (s > nblk) s = nblk;
  if (s < 1) s = 1;
  return (int)s;
}

// The library's split count with per-sequence lengths: four times the dense choice
// (capped by the blocks of a full sequence and 4096).  Every sequence is split S ways,
// so a short one has short items; with about four items per wave the persistent grid
// evens the lengths out better than with one.
int auto_splits_seq(const kvq_config& c) {
  int64_t s = (int64_t)auto_splits(c) * 4;
  const int64_t nblk = c.capacity / c.k_block;
  if (s > nblk) s = nblk;
  if (s > 4096) s = 4096;
  return (int)(s < 1 ? 1 : s);
}

// Splits per (b, kv-head) for a chunk of nq queries: about two work items per SIMD of
// an MI355X (256 CUs x 4) over the row tiles of 16, in multiples of 4 (the waves of a
// matrix-core workgroup), without splitting a sequence below one block per split.
int auto_chunk_splits(const kvq_config& c, int nq) {
  const int64_t rows = (int64_t)(c.q_heads / c.kv_heads) * nq;
  const int64_t units = (int64_t)c.batch * c.kv_heads * ((rows + 15) / 16);
  int64_t s = (2048 + units - 1) / units;
  s = (s + 3) / 4 * 4;
  const int64_t nblk = c.capacity / c.k_block;
  if (s > nblk) s = nblk;
  if (s > 4096) s = 4096;
  if (s < 1) s = 1;
  return (int)s;
}

constexpr int32_t kMaxChunk = 1024;

// Longest cache (in quantized blocks per sequence) that a decode step takes in one launch:
// one block per wave of its workgroup.  (With two per wave the split kernels are faster.)
constexpr int64_t kStepOneLaunchBlocks = 4;

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_ECAPACITY: return "cache capacity exceeded";
    case KVQ_EWORKSPACE: return "workspace too small";
    case KVQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

kvq_status kvq_cache_layout(const kvq_config* cfg, kvq_layout* out) {
  if (!out) return KVQ_EINVAL;
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  const kvq_config& c = *cfg;
  const size_t BH = (size_t)c.batch * c.kv_heads, D = c.head_dim, T = c.capacity;
  const size_t nblk = T / c.k_block, ko = kvq::host_kout(c);
  memset(out, 0, sizeof *out);
  out->k_codes = BH * T * D * c.k_bits / 8;
  if (c.k_mode == 0) {
    out->k_scale = BH * nblk * D * 2;
    out->k_zero = out->k_scale;
  } else if (c.k_mode == 1) {
    out->k_lut = (size_t)c.kv_heads * D * ((size_t)1 << c.k_bits) * 2;
  }
  out->k_tail = BH * c.k_block * D * 2;
  out->v_codes = BH * T * D * c.v_bits / 8;
  if (c.v_mode == 0) {
    out->v_scale = BH * T * (D / c.v_group) * 2;
    out->v_zero = out->v_scale;
  } else if (c.v_mode == 1) {
    out->v_lut = (size_t)c.kv_heads * D * ((size_t)1 << c.v_bits) * 2;
  }
  out->v_tail = out->k_tail;
  if (ko) {
    out->k_rowptr = BH * (T + 1) * 4;
    out->k_col = BH * T * ko;
    out->k_val = BH * T * ko * 2;
    out->v_rowptr = out->k_rowptr;
    out->v_col = out->k_col;
    out->v_val = out->k_val;
  }
  out->rope = ((size_t)c.k_block + nblk) * (D / 2) * 2 * 4;
  const size_t R = kvq::keep_count(c);
  out->k_keep_idx = BH * nblk * R;
  out->k_keep_val = BH * nblk * R * D * 2;
  return KVQ_OK;
}

kvq_status kvq_paged_layout(const kvq_config* cfg, int32_t num_blocks, kvq_layout* out) {
  kvq_status st = kvq_cache_layout(cfg, out);
  if (st != KVQ_OK) return st;
  if (num_blocks < 1 || (int64_t)num_blocks * cfg->kv_heads >= ((int64_t)1 << 31)) return KVQ_EINVAL;
  // per slot as in the dense layout, num_blocks * kv_heads slots instead of
  // batch * kv_heads * (T / Bk); row pointers per slot
  const size_t dense_slots = (size_t)cfg->batch * cfg->kv_heads * (cfg->capacity / cfg->k_block);
  const size_t slots = (size_t)num_blocks * cfg->kv_heads;
  auto per = [&](size_t& x) { x = x / dense_slots * slots; };
  per(out->k_codes);
  per(out->k_scale);
  per(out->k_zero);
  per(out->v_codes);
  per(out->v_scale);
  per(out->v_zero);
  per(out->k_col);
  per(out->k_val);
  per(out->v_col);
  per(out->v_val);
  per(out->k_keep_idx);
  per(out->k_keep_val);
  if (out->k_rowptr) {
    out->k_rowptr = slots * (cfg->k_block + 1) * 4;
    out->v_rowptr = out->k_rowptr;
  }
  return KVQ_OK;
}

kvq_status kvq_cache_init(kvq_cache* cache, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  st = from_hip(kvq::launch_rope_init(*cache, (hipStream_t)stream));
  if (st == KVQ_OK && per_sequence(cache)) st = from_hip(kvq::launch_seq_lens_set(*cache, 0, (hipStream_t)stream));
  if (st != KVQ_OK) return st;
  cache->length = 0;
  if (per_sequence(cache))
    for (int b = 0; b < cache->cfg.batch; ++b) cache->seq_lens_host[b] = 0;
  return st;
}

kvq_status kvq_quantize_append_seqs(kvq_cache* cache, const void* k_new, const void* v_new, int64_t n_max,
                                    const int64_t* n_new_host, const int64_t* n_new_dev, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (!per_sequence(cache) || !n_new_host || !n_new_dev || n_max < 0) return KVQ_EINVAL;
  bool any = false;
  for (int b = 0; b < cache->cfg.batch; ++b) {
    if (n_new_host[b] < 0 || n_new_host[b] > n_max) return KVQ_EINVAL;
    any = any || n_new_host[b] > 0;
  }
  if (!any) return KVQ_OK;
  if (!k_new || !v_new) return KVQ_EINVAL;
  return append_per_sequence(cache, (const uint16_t*)k_new, (const uint16_t*)v_new, n_max, n_new_host, n_new_dev,
                             (hipStream_t)stream);
}

kvq_status kvq_quantize_append(kvq_cache* cache, const void* k_new, const void* v_new,
                               int64_t n_new, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (n_new < 0) return KVQ_EINVAL;
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new) return KVQ_EINVAL;
  const kvq_config& c = cache->cfg;
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* kn = (const uint16_t*)k_new;
  const uint16_t* vn = (const uint16_t*)v_new;
  if (per_sequence(cache)) return append_per_sequence(cache, kn, vn, n_new, nullptr, nullptr, s);
  const int64_t L0 = cache->length, L1 = L0 + n_new, Bk = c.k_block;
  if (L1 > c.capacity) return KVQ_ECAPACITY;
  const int64_t nf0 = L0 / Bk, nf1 = L1 / Bk;
  if (nf1 > nf0) {
    st = from_hip(kvq::launch_quantize(*cache, kn, vn, L0, n_new, nf0, nf1 - nf0, s));
    if (st != KVQ_OK) return st;
  }
  // the newest L1 % Bk tokens stay unquantized in the tails
  const int64_t rem = L1 - nf1 * Bk;
  if (rem > 0) {
    const int64_t src0 = n_new - (nf1 > nf0 ? rem : n_new);
    const int64_t dst0 = nf1 > nf0 ? 0 : L0 - nf0 * Bk;
    st = from_hip(kvq::launch_tail_copy(*cache, kn, vn, n_new, src0, dst0, s));
    if (st != KVQ_OK) return st;
  }
  cache->length = L1;
  return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t num_splits) {
  if (check_cache(cache) != KVQ_OK || num_splits < 0) return 0;
  const kvq_config& c = cache->cfg;
  const int S = num_splits ? num_splits : (per_sequence(cache) ? auto_splits_seq(c) : auto_splits(c));
  return (size_t)c.batch * c.q_heads * S * (c.head_dim + 2) * sizeof(float);
}

kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q, int64_t q_pos, float* out,
                                void* ws, size_t ws_bytes, int32_t num_splits, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (!q || !out || num_splits < 0) return KVQ_EINVAL;
  st = check_decode_pos(cache, q_pos);
  if (st != KVQ_OK) return st;
  const kvq_config& c = cache->cfg;
  const int S = num_splits ? num_splits : (per_sequence(cache) ? auto_splits_seq(c) : auto_splits(c));
  if (S > 4096) return KVQ_EINVAL;
  const size_t need = (size_t)c.batch * c.q_heads * S * (c.head_dim + 2) * sizeof(float);
  if (!ws || ws_bytes < need) return KVQ_EWORKSPACE;
  return from_hip(kvq::launch_decode(*cache, (const uint16_t*)q, q_pos, out, (float*)ws, S,
                                     (hipStream_t)stream));
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q, int64_t q_pos, float* out,
                                        int32_t num_splits, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (!q || !out || num_splits < 0) return KVQ_EINVAL;
  st = check_decode_pos(cache, q_pos);
  if (st != KVQ_OK) return st;
  const kvq_config& c = cache->cfg;
  const int S = num_splits ? num_splits : (per_sequence(cache) ? auto_splits_seq(c) : auto_splits(c));
  if (S > 4096) return KVQ_EINVAL;
  const size_t need = (size_t)c.batch * c.q_heads * S * (c.head_dim + 2) * sizeof(float);
  if (need > kNoallocScratchBytes) return KVQ_EWORKSPACE;
  float* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != KVQ_OK) return st;
  return from_hip(kvq::launch_decode(*cache, (const uint16_t*)q, q_pos, out, ws, S,
                                     (hipStream_t)stream));
}

kvq_status kvq_decode_step(kvq_cache* cache, const void* k_new, const void* v_new, const void* q, float* out,
                           void* ws, size_t ws_bytes, int32_t num_splits, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (!k_new || !v_new || !q || !out || num_splits < 0 || num_splits > 4096) return KVQ_EINVAL;
  if (per_sequence(cache)) return KVQ_EUNSUPPORTED;
  const kvq_config& c = cache->cfg;
  const int64_t L0 = cache->length, L1 = L0 + 1, Bk = c.k_block;
  if (L1 > c.capacity) return KVQ_ECAPACITY;
  const int S = num_splits ? num_splits : auto_splits(c);
  const size_t need = (size_t)c.batch * c.q_heads * S * (c.head_dim + 2) * sizeof(float);
  if (!ws || ws_bytes < need) return KVQ_EWORKSPACE;
  // one launch while the cache is short enough that launches, not bandwidth, set the cost
  const bool one_launch =
      num_splits == 0 && L1 / Bk <= kStepOneLaunchBlocks && kvq::decode_step_prefers_one_launch(*cache);
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* kn = (const uint16_t*)k_new;
  const uint16_t* vn = (const uint16_t*)v_new;
  int jnew = (int)(L0 % Bk);
  if (L1 % Bk == 0) {  // the token completes a block: quantize it (tail + token) first
    st = from_hip(kvq::launch_quantize(*cache, kn, vn, L0, 1, L0 / Bk, 1, s));
    if (st != KVQ_OK) return st;
    jnew = -1;
  }
  kvq_cache next = *cache;
  next.length = L1;
  st = from_hip(kvq::launch_decode_step(next, (const uint16_t*)q, kn, vn, jnew, out, (float*)ws,
                                        one_launch ? 0 : S, s));
  if (st != KVQ_OK) return st;
  cache->length = L1;
  return KVQ_OK;
}

size_t kvq_chunk_workspace_bytes(const kvq_cache* cache, int32_t nq, int32_t num_splits) {
  if (check_cache(cache) != KVQ_OK || num_splits < 0 || nq < 1 || nq > kMaxChunk) return 0;
  const kvq_config& c = cache->cfg;
  const int S = num_splits ? num_splits : auto_chunk_splits(c, nq);
  return (size_t)c.batch * c.q_heads * nq * S * (c.head_dim + 2) * sizeof(float);
}

kvq_status kvq_chunk_attention(const kvq_cache* cache, const void* q, int32_t nq, int64_t q_pos, float* out,
                               void* ws, size_t ws_bytes, int32_t num_splits, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (per_sequence(cache)) return KVQ_EUNSUPPORTED;
  if (!q || !out || q_pos < 0 || num_splits < 0 || cache->length == 0) return KVQ_EINVAL;
  if (nq < 1 || nq > kMaxChunk || q_pos > (int64_t)1 << 40) return KVQ_EINVAL;
  const kvq_config& c = cache->cfg;
  const int S = num_splits ? num_splits : auto_chunk_splits(c, nq);
  if (S > 4096) return KVQ_EINVAL;
  const size_t need = (size_t)c.batch * c.q_heads * nq * S * (c.head_dim + 2) * sizeof(float);
  if (!ws || ws_bytes < need) return KVQ_EWORKSPACE;
  return from_hip(kvq::launch_chunk(*cache, (const uint16_t*)q, nq, q_pos, out, (float*)ws, S,
                                    (hipStream_t)stream));
}

kvq_status kvq_dequantize(const kvq_cache* cache, int32_t which, int64_t t0, int64_t t1, float* out,
                          void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (per_sequence(cache)) return KVQ_EUNSUPPORTED;
  if ((which != 0 && which != 1) || t0 < 0 || t1 < t0 || t1 > cache->length) return KVQ_EINVAL;
  if (t1 == t0) return KVQ_OK;
  if (!out) return KVQ_EINVAL;
  return from_hip(kvq::launch_dequantize(*cache, which, t0, t1, out, (hipStream_t)stream));
}

}  // extern "C"
