/*
 * kvq.h -- C ABI of libkvq: 2/3/4-bit KV-cache quantization and single-query decode
 * attention computed directly over the packed cache, on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, address):
 *   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
 *   [TQ]   "TurboQuant：突破大模型推理瓶颈的KVCache量化技术解析", mlqm.cn/news/1002276
 *   [UQ]   "大模型长上下文推理优化：4-bit KV Cache量化技术解析与部署实践", mlqm.cn/news/1064729
 *
 * The three operations follow the problem the pages pose: quantize keys and values
 * when they enter the cache, keeping per-block scale and zero-point metadata
 * ([KVC3] "Quanto 的量化原理"; [TQ] section 4.2), accumulating tokens by block
 * ([UQ] section 4.2); and either dequantize or compute attention directly on the
 * quantized form when it is read ([KVC3] "Pre-RoPE Key Quantization" and the
 * custom kernels of "Q-Norm 与其他细节"; [UQ] section 4.2 on fusing dequantization
 * into attention).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Memory: the caller allocates every device buffer (sizes from kvq_cache_layout)
 *   and frees it; the library allocates no device memory and keeps no state between
 *   calls.  Pointers named *device* must be device (or managed) memory of the GPU
 *   that is current on the calling thread.
 * - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Every call only enqueues work on it and returns; nothing synchronises the device.
 * - Errors: arguments are checked on the host before anything is enqueued.  On any
 *   error return nothing has been enqueued and the cache (including `length`) is
 *   unchanged.  KVQ_EHIP means a launch failed after checking; the cache contents are
 *   then undefined.  No C++ exception crosses this interface.
 * - Inputs must be finite; the library does not scan for NaN or Inf.
 * - Calls on different caches are independent; concurrent calls on one cache are
 *   undefined.
 *
 * fp16 values are IEEE binary16 bit patterns (uint16_t).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvq_status;
#define KVQ_OK 0
#define KVQ_EINVAL (-1)        /* malformed arguments or descriptor                 */
#define KVQ_EUNSUPPORTED (-2)  /* well-formed, but outside what the kernels build   */
#define KVQ_ECAPACITY (-3)     /* append would exceed capacity; nothing written      */
#define KVQ_EWORKSPACE (-4)    /* workspace too small                                */
#define KVQ_EHIP (-5)          /* a HIP launch or query failed                       */

/* Immutable description of one layer's cache.
 *
 * Keys: quantized before RoPE ([KVC3] "Pre-RoPE Key Quantization").
 *   k_mode 0: uniform asymmetric, one fp16 scale and zero-point per channel per
 *             block of k_block tokens ([KVC3] "Per-Channel Key Quantization").
 *   k_mode 1: per-channel non-uniform codebook of 2^k_bits sorted fp16 entries,
 *             supplied by the caller ([KVC3] "Non-Uniform KV Cache Quantization").
 *   k_mode 2: FP8 cache ([UQ] section 2.1): every key element cast to OCP E4M3 (4
 *             exponent bits, bias 7, 3 mantissa bits, largest finite 448), nearest with
 *             ties to even, saturating at +-448; requires v_mode 2 and k_bits = v_bits
 *             = 8.  The byte is the code; no metadata.
 * Values:
 *   v_mode 0: uniform asymmetric per token over groups of v_group channels, one fp16
 *             scale and zero-point per group ([KVC3] "Quanto 的量化原理").
 *   v_mode 1: per-channel non-uniform codebook of 2^v_bits sorted fp16 entries per
 *             (kv head, channel), supplied by the caller: the page applies the
 *             non-uniform format to the Value cache first ([KVC3] "Non-Uniform KV Cache
 *             Quantization"); a codebook of log-spaced levels is the log quantization of
 *             [TQ] section 3.3.  The code is the nearest entry, decided at the fp32
 *             midpoints, ties to the lower code (as for codebook keys).
 *   v_mode 2: FP8 values, cast to E4M3 like the keys of k_mode 2 (the two go together).
 * clip_quantile q > 0: before the statistics, every dense value of a block is
 *   clipped to [-t, t], t = the q-quantile of |x| over that block's k_block x
 *   head_dim elements of the same tensor (exact order statistics, linear
 *   interpolation), as the percentile clip of [UQ] section 4.2.  0 disables.
 * outlier_pct p > 0: in every token vector of K and of V, the ceil(p*head_dim/100)
 *   elements of largest |x| are kept exactly as fp16 in a per-token CSR and take
 *   no part in the statistics ([KVC3] "Per-Vector Dense-and-Sparse Quantization").
 * rope_theta: base of the rotary embedding applied to keys and the query at read
 *   time (rotate-half pairs (i, i + head_dim/2), angle pos * theta^(-2i/head_dim)).
 * keep_pct p > 0: in every quantized block the R = ceil(p*k_block/100) key vectors of
 *   largest squared L2 norm (the fp16 values squared exactly in fp64 and added in
 *   channel order; ties to the lower token) are kept exactly as fp16 and take no part
 *   in the block's statistics (code 0 is stored for them): the norm-based importance
 *   and high-precision retention of [TQ] sections 3.2 and 6.1.  Values are quantized
 *   as usual.
 *
 * Supported by the kernels: head_dim in {64, 128}; k_bits in {2, 3, 4} (k_mode 0 or
 * 1); v_bits in {2, 4}; v_group in {16, 32, 64, 128} dividing head_dim; k_block in
 * {64, 128}; capacity a positive multiple of k_block below 2^31; q_heads a multiple of
 * kv_heads with q_heads/kv_heads <= 8; clip_quantile in [0, 1); outlier_pct in
 * [0, 100] with ceil(p*head_dim/100) <= 4; rope_theta > 1; keep_pct in [0, 100] with
 * R <= 16, and only with uniform keys (k_mode 0), no outliers and no clipping; v_mode in
 * {0, 1, 2}, 1 and 2 only without outliers and clipping; the FP8 cache (k_mode 2, v_mode
 * 2, 8 bits) without kept keys.
 */
typedef struct {
  int32_t batch, q_heads, kv_heads, head_dim, capacity;
  int32_t k_bits, k_mode, k_block;
  int32_t v_bits, v_group;
  float clip_quantile;
  int32_t outlier_pct;
  float rope_theta;
  int32_t keep_pct;
  int32_t v_mode;
} kvq_config;

/* Byte size of each buffer of a cache; 0 = buffer not used by this configuration. */
typedef struct {
  size_t k_codes, k_scale, k_zero, k_lut, k_tail;
  size_t v_codes, v_scale, v_zero, v_tail;
  size_t k_rowptr, k_col, k_val, v_rowptr, v_col, v_val;
  size_t rope;
  size_t k_keep_idx, k_keep_val;
  size_t v_lut;
} kvq_layout;

/* A cache: caller-owned device buffers plus the host-side token count.
 * Shapes, with BH = batch * kv_heads in (b, h) row-major order, T = capacity,
 * D = head_dim, Bk = k_block, ko = outliers per vector (0 if off):
 *
 *  k_codes  u8   [BH][T][D*k_bits/8]  one packed row per token.  Row element e,
 *                 at bits [e*k_bits, (e+1)*k_bits) of the little-endian row, LSB
 *                 first (a 3-bit code may straddle two bytes), holds channel
 *                 (e >> 1) + (e & 1) * D/2: each rotary pair sits side by side.
 *  k_scale  fp16 [BH][T/Bk][D]        uniform keys: scale per block and channel.
 *  k_zero   fp16 [BH][T/Bk][D]        uniform keys: zero-point (x = c*scale + zero).
 *  k_lut    fp16 [kv_heads][D][2^k_bits] codebook keys: input, sorted ascending.
 *  k_tail   fp16 [BH][Bk][D]          the length % Bk newest keys, unquantized.
 *  v_codes  u32  [BH][T/(32/v_bits)][D] words: word (t / tpw, d), tpw = 32/v_bits,
 *                 holds the codes of channel d for tpw consecutive tokens; token t
 *                 at bits [(t % tpw)*v_bits, ...).
 *  v_scale  fp16 [BH][T][D/v_group]   uniform values only.
 *  v_zero   fp16 [BH][T][D/v_group]   uniform values only.
 *  v_lut    fp16 [kv_heads][D][2^v_bits] codebook values: input, sorted ascending.
 *  v_tail   fp16 [BH][Bk][D]
 *  k_rowptr i32  [BH][T+1]            CSR row pointers of key outliers; for every
 *                 quantized token rowptr[t+1] - rowptr[t] == ko and rowptr[0] == 0.
 *  k_col    u8   [BH][T*ko]           outlier channels, ascending within a token.
 *  k_val    fp16 [BH][T*ko]           outlier values, exact input bits.
 *  v_rowptr, v_col, v_val: the same for values.
 *  rope     f32  [Bk][D/2][2] cos/sin(j * f_i), then [T/Bk][D/2][2] cos/sin(n*Bk*f_i),
 *                 with f_i = theta^(-2i/D); filled by kvq_cache_init.
 *  k_keep_idx u8   [BH][T/Bk][R]     keep_pct > 0: the kept tokens' offsets in the
 *                 block, ascending.
 *  k_keep_val fp16 [BH][T/Bk][R][D]  their key vectors, exact input bits.
 *
 * Tokens [0, floor(length/Bk)*Bk) are quantized; the rest live in the tails.
 * At a quantized position that holds an outlier the stored code is 0; readers
 * use the CSR value there.
 *
 * Every buffer above except the tails, k_lut, rope and the row pointers is an array of
 * per-block slots: block n of (b, h) is slot g = (b * kv_heads + h) * (T / Bk) + n, and
 * the slot's part of a buffer is its Bk tokens' rows (k_codes, v_codes, v_scale,
 * v_zero, k_col/k_val and v_col/v_val, the latter Bk * ko entries), its D entries
 * (k_scale, k_zero) or its R kept keys (k_keep_idx, k_keep_val).
 *
 * Paged layout (block_table != NULL), for the continuous batching and paged cache
 * management that [TQ] sections 5.2 and 5.3 name as the serving context of a quantized
 * cache.  The quantized blocks of all sequences live in one pool of
 * num_blocks physical blocks; sequence b's logical block n is physical block
 * p = block_table[b * (T / Bk) + n], and its slot for kv head h is g = p * kv_heads + h
 * (the buffers hold num_blocks * kv_heads slots; kvq_paged_layout gives their sizes).
 * Each sequence has its own length: seq_lens (device, [batch]) is what the kernels read,
 * seq_lens_host (host, [batch]) what the host sequences the launches by; the library
 * advances both (the device copy stream-ordered).  `length` is unused.  The row
 * pointers are per slot, [num_blocks * kv_heads][Bk + 1], local to the slot's Bk tokens.
 * The tails stay per sequence, [batch][kv_heads][Bk][D].  T = capacity is the most
 * tokens one sequence may hold (the table's row length is T / Bk).  The caller owns
 * the table: every block a sequence holds (n < seq_lens[b] / Bk, and the blocks an
 * append completes) must map to a distinct physical block; the kernels clamp an entry
 * into [0, num_blocks), so a wrong table gives wrong results but no fault.
 */
typedef struct {
  kvq_config cfg;
  int64_t length;
  void *k_codes;
  uint16_t *k_scale, *k_zero;
  const uint16_t *k_lut;
  uint16_t *k_tail;
  void *v_codes;
  uint16_t *v_scale, *v_zero, *v_tail;
  int32_t *k_rowptr;
  uint8_t *k_col;
  uint16_t *k_val;
  int32_t *v_rowptr;
  uint8_t *v_col;
  uint16_t *v_val;
  float *rope;
  uint8_t *k_keep_idx;
  uint16_t *k_keep_val;
  const uint16_t *v_lut;
  /* paged layout (see above); all NULL / 0 for the dense layout */
  const int32_t *block_table;
  int32_t num_blocks;
  int64_t *seq_lens;
  int64_t *seq_lens_host;
} kvq_cache;

/* Text for a status code (static storage; never NULL).  No passage of the pages defines
 * an error model: the codes are this interface's own, so that a framework that embeds
 * the cache (the integration [TQ] section 5.3 says the attention and cache management
 * must undergo) can report why a call was refused. */
const char *kvq_status_string(kvq_status s);

/* Validate `cfg` and report the byte size of every buffer.  Host only; touches no
 * GPU.  KVQ_EINVAL for malformed values, KVQ_EUNSUPPORTED for well-formed values the
 * kernels do not build.  The total follows the cache-size formula of [TQ] section 2.1
 * with the packed widths of [KVC3] "前言" (4 bits instead of 16). */
kvq_status kvq_cache_layout(const kvq_config *cfg, kvq_layout *out);

/* The buffer sizes of a paged cache whose pool holds num_blocks physical blocks (per
 * slot as kvq_cache_layout's, times num_blocks * kv_heads slots; row pointers
 * [slots][Bk + 1]; tails, k_lut and rope as in the dense layout).  Host only.
 * KVQ_EINVAL also for num_blocks < 1 or num_blocks * kv_heads >= 2^31. */
kvq_status kvq_paged_layout(const kvq_config *cfg, int32_t num_blocks, kvq_layout *out);

/* Prepare an empty cache: validates the descriptor and its buffer pointers,
 * fills `rope` (angles evaluated in fp64) and sets length = 0.  Enqueued on `stream`.
 * The pages apply RoPE to the keys after dequantization ([KVC3] "Pre-RoPE Key
 * Quantization"); `rope` holds the cos/sin of those angles once per cache, in a
 * caller-owned buffer like every other buffer, so that no decode evaluates them. */
kvq_status kvq_cache_init(kvq_cache *cache, void *stream);

/* Append n_new tokens for every (b, kv-head): k_new, v_new are *device* fp16
 * [batch][kv_heads][n_new][head_dim], keys pre-RoPE.  Every token block that
 * becomes complete (absolute positions [j*Bk, (j+1)*Bk)) is quantized from its
 * tokens (old tail + new); the remaining newest tokens go to the tails, as in the
 * block accumulation of [UQ] section 4.2.  `length` grows by n_new on the host at
 * enqueue time.  n_new == 0 is a no-op.  KVQ_ECAPACITY if length + n_new > capacity. */
kvq_status kvq_quantize_append(kvq_cache *cache, const void *k_new, const void *v_new,
                               int64_t n_new, void *stream);

/* Append a different number of tokens to each sequence of a cache with per-sequence
 * lengths (seq_lens set; dense or paged): sequence b takes the first n_new_host[b]
 * rows of k_new[b], v_new[b] (*device* fp16 [batch][kv_heads][n_max][head_dim], keys
 * pre-RoPE; rows past a sequence's count are not read).  This is one step of continuous
 * batching ([TQ] section 5.2): sequences in prefill take many tokens, sequences in
 * decode one, finished ones none.  n_new_dev: *device* int64 [batch], equal to
 * n_new_host (the kernels read it; the host copy sizes the launches).  Blocks are
 * quantized and tails kept per sequence as in kvq_quantize_append; both length copies
 * advance by the counts.  KVQ_EINVAL for a cache without per-sequence lengths, a count
 * outside [0, n_max] or null pointers, KVQ_ECAPACITY if a sequence would exceed
 * capacity (nothing is written then). */
kvq_status kvq_quantize_append_seqs(kvq_cache *cache, const void *k_new, const void *v_new, int64_t n_max,
                                    const int64_t *n_new_host, const int64_t *n_new_dev, void *stream);

/* Bytes of device workspace kvq_decode_attention needs for `num_splits` splits of
 * the cache per (b, kv-head) (0 = the library's choice for this cache; at most
 * 4096): one (max, sum, output) partial of head_dim + 2 floats per (b, q-head, split),
 * B * q_heads * splits * (head_dim + 2) * 4 bytes.  The split-K decode reads the
 * packed cache once and keeps only these partials as intermediate state, in the
 * FlashAttention manner [TQ] section 5.2 pairs with the quantized cache.  With
 * per-sequence lengths the library's choice is four times the dense one (more, shorter
 * work items even out the different lengths).  Host only; returns 0 for an invalid
 * cache or a negative split count. */
size_t kvq_decode_workspace_bytes(const kvq_cache *cache, int32_t num_splits);

/* Single-query decode attention over the whole cache:
 *   out[b][hq] = softmax_t( RoPE(q[b][hq], q_pos) . RoPE(k_hat[b][h][t], t) / sqrt(D) ) v_hat[b][h][t]
 * with h = hq / (q_heads/kv_heads), t in [0, length), k_hat and v_hat the
 * dequantized keys and values (outliers and tails exact).  RoPE is applied to the
 * keys after dequantization ([KVC3] "Pre-RoPE Key Quantization").
 * q: *device* fp16 [batch][q_heads][head_dim], pre-RoPE.  out: *device* fp32
 * [batch][q_heads][head_dim].  ws: *device* workspace of ws_bytes >=
 * kvq_decode_workspace_bytes(cache, num_splits).  q_pos >= 0 (usually length-1).
 * The result does not depend on num_splits beyond fp32 rounding and is bitwise
 * reproducible for a fixed num_splits.  KVQ_EINVAL if length == 0 or num_splits is
 * negative or above 4096. */
kvq_status kvq_decode_attention(const kvq_cache *cache, const void *q, int64_t q_pos,
                                float *out, void *ws, size_t ws_bytes, int32_t num_splits,
                                void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same decode as
 * kvq_decode_attention, with the split partials kept in a library-owned device array
 * of KVQ_NOALLOC_SCRATCH_BYTES per GPU (B * q_heads * splits * (head_dim + 2) * 4 bytes
 * must fit: KVQ_EWORKSPACE otherwise) instead of a caller workspace.  The array is
 * set up on a device at the first call made with that device current and held until
 * the process ends; this call allocates nothing.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (e.g. on two streams) race and give
 * undefined results.  Same arguments, results and errors as kvq_decode_attention
 * otherwise (bitwise the same output for the same num_splits). */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_cache *cache, const void *q, int64_t q_pos,
                                        float *out, int32_t num_splits, void *stream);

/* One decode step with its token, fused: append one new token per sequence and attend
 * with the query at the token's position over the whole cache, the token included:
 *   the same results as kvq_quantize_append(cache, k_new, v_new, 1) followed by
 *   kvq_decode_attention(cache, q, length - 1, ...) (up to fp32 rounding).
 * The pages name per-head launches and the quantize/dequantize round trips as costs of
 * the quantized cache and fusion as their cure ([TQ] sections 5.1 and 6.3).  The token
 * never takes a launch of its own: the attention reads it from k_new/v_new and one of
 * its kernels stores it into the fp16 tail.  When it completes a block, that block is
 * quantized first (one launch, as by kvq_quantize_append).
 * num_splits == 0 (the library's choice): the split kernels of kvq_decode_attention with
 * the library's split count (two launches), except for a short cache (at most 4
 * quantized blocks per sequence) in a configuration that none of the tuned decode kernels
 * covers: that takes ONE launch, one workgroup per (b, kv-head) whose waves split the
 * cache and merge in LDS.  (Where a tuned kernel applies, it and the merge launch take
 * less time than the one generic launch, even at 256 tokens.)  num_splits > 0: the two
 * launches with that many splits.
 * ws: device workspace of at least kvq_decode_workspace_bytes(cache, num_splits) bytes
 * (the same as kvq_decode_attention's; the one-launch path does not touch it).
 * k_new, v_new: *device* fp16 [batch][kv_heads][head_dim], keys pre-RoPE; q: *device*
 * fp16 [batch][q_heads][head_dim]; out: *device* fp32 [batch][q_heads][head_dim].
 * `length` grows by one on the host at enqueue time.  KVQ_ECAPACITY if the cache is
 * full, KVQ_EWORKSPACE for a workspace that is too small, KVQ_EINVAL for a split count
 * that is negative or above 4096; on any error the cache is left unchanged. */
kvq_status kvq_decode_step(kvq_cache *cache, const void *k_new, const void *v_new, const void *q,
                           float *out, void *ws, size_t ws_bytes, int32_t num_splits,
                           void *stream);

/* Bytes of device workspace kvq_chunk_attention needs for a chunk of nq queries and
 * `num_splits` splits per (b, kv-head) (0 = the library's choice; at most 4096): one
 * (max, sum, output) partial of head_dim + 2 floats per (b, q-head, query, split),
 * B * q_heads * nq * splits * (head_dim + 2) * 4 bytes, in the FlashAttention manner
 * of [TQ] section 5.2.  Host only; returns 0 for an invalid cache, nq outside
 * [1, 1024] or a negative split count. */
size_t kvq_chunk_workspace_bytes(const kvq_cache *cache, int32_t nq, int32_t num_splits);

/* Causal attention of a chunk of nq consecutive query tokens over the cache: a
 * prefill chunk, or the draft tokens of a speculative-verification step ([UQ]
 * section 5.1 counts first-token latency among the costs a deployment measures).
 * Query j sits at position q_pos + j and sees the cache tokens t <= q_pos + j:
 *   out[b][hq][j] = softmax_{t < n_j}( RoPE(q[b][hq][j], q_pos + j) . RoPE(k_hat[b][h][t], t) / sqrt(D) ) v_hat[b][h][t],
 *   n_j = min(q_pos + j + 1, length),
 * with h = hq / (q_heads/kv_heads) and k_hat, v_hat as in kvq_decode_attention.  The
 * usual call appends the chunk's own keys and values first (kvq_quantize_append) and
 * passes q_pos = length - nq.  With nq = 1 and q_pos = length - 1 this is the decode
 * step.  q: *device* fp16 [batch][q_heads][nq][head_dim], pre-RoPE.  out: *device*
 * fp32 [batch][q_heads][nq][head_dim].  ws: *device* workspace of ws_bytes >=
 * kvq_chunk_workspace_bytes(cache, nq, num_splits).  The result does not depend on
 * num_splits beyond fp32 rounding.  KVQ_EINVAL if length == 0, nq outside [1, 1024],
 * q_pos < 0, or num_splits negative or above 4096. */
kvq_status kvq_chunk_attention(const kvq_cache *cache, const void *q, int32_t nq, int64_t q_pos,
                               float *out, void *ws, size_t ws_bytes, int32_t num_splits,
                               void *stream);

/* Dequantize tokens [t0, t1) of keys (which = 0) or values (which = 1) into *device*
 * fp32 out [batch][kv_heads][t1-t0][head_dim], pre-RoPE: x = fmaf(c, scale, zero) or
 * the codebook entry, outlier positions and tail tokens exact.  This is the
 * "dequantize before use" read of [TQ] section 4.2 and the scale/zero-point
 * reconstruction of [KVC3] "Quanto 的量化原理", for callers that want the values
 * rather than attention over them.  0 <= t0 <= t1 <= length; t0 == t1 is a no-op;
 * KVQ_EINVAL for a bad range or `which`. */
kvq_status kvq_dequantize(const kvq_cache *cache, int32_t which, int64_t t0, int64_t t1,
                          float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
