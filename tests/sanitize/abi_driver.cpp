// Runs the host side of the C ABI (argument checks, buffer sizing, split choice, error
// returns) under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU: the
// kernel launchers are replaced by stubs that report a launch failure, so every path
// that passes its checks ends in KVQ_EHIP with the cache untouched.  Exit status 0 =
// every expectation held and the sanitizers stayed silent.
#include <stdio.h>
#include <string.h>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {
hipError_t launch_rope_init(const kvq_cache&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quantize(const kvq_cache&, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t,
                           hipStream_t, const int64_t*) {
  return hipErrorNotSupported;
}
hipError_t launch_tail_copy(const kvq_cache&, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t,
                            hipStream_t, const int64_t*) {
  return hipErrorNotSupported;
}
hipError_t launch_decode(const kvq_cache&, const uint16_t*, int64_t, float*, float*, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_dequantize(const kvq_cache&, int, int64_t, int64_t, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_chunk(const kvq_cache&, const uint16_t*, int, int64_t, float*, float*, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode_step(const kvq_cache&, const uint16_t*, const uint16_t*, const uint16_t*, int, float*,
                              float*, int, hipStream_t) {
  return hipErrorNotSupported;
}
bool decode_step_prefers_one_launch(const kvq_cache&) { return true; }
hipError_t launch_seq_lens_add(const kvq_cache&, int64_t, hipStream_t, const int64_t*) { return hipErrorNotSupported; }
hipError_t launch_seq_lens_set(const kvq_cache&, int64_t, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kvq

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static kvq_config base() {
  kvq_config c;
  memset(&c, 0, sizeof c);
  c.batch = 2; c.q_heads = 8; c.kv_heads = 2; c.head_dim = 128; c.capacity = 1024;
  c.k_bits = 4; c.k_mode = 0; c.k_block = 128; c.v_bits = 4; c.v_group = 128;
  c.clip_quantile = 0.99f; c.outlier_pct = 1; c.rope_theta = 10000.0f;
  return c;
}

// A descriptor whose buffers are distinct non-null addresses that are never touched.
static kvq_cache fake_cache(const kvq_config& c, int64_t length) {
  kvq_cache k;
  memset(&k, 0, sizeof k);
  k.cfg = c;
  k.length = length;
  kvq_layout lay;
  if (kvq_cache_layout(&c, &lay) != KVQ_OK) return k;
  uintptr_t a = 0x10000;
  auto p = [&](size_t n) { a += 0x1000; return n ? (void*)a : nullptr; };
  k.k_codes = p(lay.k_codes); k.k_scale = (uint16_t*)p(lay.k_scale); k.k_zero = (uint16_t*)p(lay.k_zero);
  k.k_lut = (const uint16_t*)p(lay.k_lut); k.k_tail = (uint16_t*)p(lay.k_tail); k.v_codes = p(lay.v_codes);
  k.v_scale = (uint16_t*)p(lay.v_scale); k.v_zero = (uint16_t*)p(lay.v_zero); k.v_tail = (uint16_t*)p(lay.v_tail);
  k.k_rowptr = (int32_t*)p(lay.k_rowptr); k.k_col = (uint8_t*)p(lay.k_col); k.k_val = (uint16_t*)p(lay.k_val);
  k.v_rowptr = (int32_t*)p(lay.v_rowptr); k.v_col = (uint8_t*)p(lay.v_col); k.v_val = (uint16_t*)p(lay.v_val);
  k.rope = (float*)p(lay.rope);
  k.k_keep_idx = (uint8_t*)p(lay.k_keep_idx); k.k_keep_val = (uint16_t*)p(lay.k_keep_val);
  k.v_lut = (const uint16_t*)p(lay.v_lut);
  return k;
}

int main() {
  for (kvq_status s = -6; s <= 1; ++s) EXPECT(kvq_status_string(s) != nullptr);
  // layout: every supported combination, and each rejected field
  kvq_layout lay;
  const int dims[] = {64, 128}, blocks[] = {64, 128}, groups[] = {16, 32, 64, 128};
  for (int D : dims)
    for (int bk : blocks)
      for (int kb = 2; kb <= 4; ++kb)
        for (int mode = 0; mode <= 1; ++mode)
          for (int vb = 2; vb <= 4; vb += 2)
            for (int g : groups) {
              kvq_config c = base();
              c.head_dim = D; c.k_block = bk; c.k_bits = kb; c.k_mode = mode; c.v_bits = vb; c.v_group = g;
              const kvq_status st = kvq_cache_layout(&c, &lay);
              EXPECT(st == (g <= D ? KVQ_OK : KVQ_EINVAL));
              if (st == KVQ_OK) EXPECT(lay.k_codes == (size_t)2 * 2 * 1024 * D * kb / 8);
            }
  struct { const char* field; int value; kvq_status want; } bad[] = {
      {"head_dim", 0, KVQ_EINVAL}, {"head_dim", 63, KVQ_EINVAL}, {"head_dim", 256, KVQ_EUNSUPPORTED},
      {"k_bits", 9, KVQ_EINVAL}, {"k_bits", 5, KVQ_EUNSUPPORTED}, {"v_bits", 3, KVQ_EUNSUPPORTED},
      {"k_block", 100, KVQ_EINVAL}, {"q_heads", 7, KVQ_EINVAL}, {"capacity", -128, KVQ_EINVAL},
      {"batch", -1, KVQ_EINVAL}, {"outlier_pct", 101, KVQ_EINVAL}, {"outlier_pct", 4, KVQ_EUNSUPPORTED}};
  for (auto& b : bad) {
    kvq_config c = base();
    if (!strcmp(b.field, "head_dim")) c.head_dim = b.value;
    if (!strcmp(b.field, "k_bits")) c.k_bits = b.value;
    if (!strcmp(b.field, "v_bits")) c.v_bits = b.value;
    if (!strcmp(b.field, "k_block")) c.k_block = b.value;
    if (!strcmp(b.field, "q_heads")) c.q_heads = b.value;
    if (!strcmp(b.field, "capacity")) c.capacity = b.value;
    if (!strcmp(b.field, "batch")) c.batch = b.value;
    if (!strcmp(b.field, "outlier_pct")) c.outlier_pct = b.value;
    EXPECT(kvq_cache_layout(&c, &lay) == b.want);
  }
  EXPECT(kvq_cache_layout(nullptr, &lay) == KVQ_EINVAL);
  {  // keys kept in fp16: count, sizes, the combinations refused
    kvq_config c = base();
    c.keep_pct = 5;  // 6.4 -> 7 per block of 128
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EUNSUPPORTED);  // with outliers and clipping
    c.outlier_pct = 0; c.clip_quantile = 0.0f;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_OK);
    EXPECT(lay.k_keep_idx == (size_t)2 * 2 * 8 * 7 && lay.k_keep_val == lay.k_keep_idx * 128 * 2);
    c.keep_pct = 13;  // 17 per block
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EUNSUPPORTED);
    c.keep_pct = -1;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EINVAL);
    c.keep_pct = 5; c.k_mode = 1;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EUNSUPPORTED);
    c.k_mode = 0;
    kvq_cache kk = fake_cache(c, 0);
    EXPECT(kvq_cache_init(&kk, nullptr) == KVQ_EHIP);
    kk.k_keep_val = nullptr;
    EXPECT(kvq_cache_init(&kk, nullptr) == KVQ_EINVAL);
  }
  {  // codebook values and the FP8 cache: sizes, the combinations refused, the buffers required
    kvq_config c = base();
    c.v_mode = 1;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EUNSUPPORTED);  // with outliers and clipping
    c.outlier_pct = 0; c.clip_quantile = 0.0f;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_OK);
    EXPECT(lay.v_scale == 0 && lay.v_zero == 0 && lay.v_lut == (size_t)2 * 128 * 16 * 2);
    kvq_cache kv = fake_cache(c, 0);
    EXPECT(kvq_cache_init(&kv, nullptr) == KVQ_EHIP);
    kv.v_lut = nullptr;
    EXPECT(kvq_cache_init(&kv, nullptr) == KVQ_EINVAL);
    c.v_mode = 3;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EINVAL);
    c.v_mode = 2;  // FP8 values need FP8 keys, 8 bits each
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EINVAL);
    c.k_mode = 2;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EINVAL);
    c.k_bits = 8; c.v_bits = 8;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_OK);
    EXPECT(lay.k_codes == (size_t)2 * 2 * 1024 * 128 && lay.v_codes == lay.k_codes);
    EXPECT(lay.k_scale == 0 && lay.k_lut == 0 && lay.v_scale == 0 && lay.v_lut == 0);
    kvq_cache kf = fake_cache(c, 0);
    EXPECT(kvq_cache_init(&kf, nullptr) == KVQ_EHIP);
    c.keep_pct = 5;
    EXPECT(kvq_cache_layout(&c, &lay) == KVQ_EUNSUPPORTED);
  }
  EXPECT(kvq_cache_layout(nullptr, nullptr) == KVQ_EINVAL);

  // init, append, decode, dequantize: checks first, then the (stubbed) launch fails
  kvq_cache k = fake_cache(base(), 0);
  EXPECT(kvq_cache_init(&k, nullptr) == KVQ_EHIP);
  k.length = 300;
  EXPECT(kvq_quantize_append(&k, (void*)0x1000, (void*)0x1000, 1000, nullptr) == KVQ_ECAPACITY);
  EXPECT(kvq_quantize_append(&k, (void*)0x1000, (void*)0x1000, -1, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_quantize_append(&k, nullptr, (void*)0x1000, 5, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_quantize_append(&k, (void*)0x1000, (void*)0x1000, 0, nullptr) == KVQ_OK);
  EXPECT(kvq_quantize_append(&k, (void*)0x1000, (void*)0x1000, 5, nullptr) == KVQ_EHIP);     // tail only
  EXPECT(kvq_quantize_append(&k, (void*)0x1000, (void*)0x1000, 500, nullptr) == KVQ_EHIP);   // blocks
  EXPECT(k.length == 300);
  const size_t ws = kvq_decode_workspace_bytes(&k, 0);
  EXPECT(ws > 0 && ws == kvq_decode_workspace_bytes(&k, 0));
  EXPECT(kvq_decode_workspace_bytes(&k, 7) == (size_t)2 * 8 * 7 * 130 * 4);
  EXPECT(kvq_decode_workspace_bytes(nullptr, 7) == 0);
  float* out = (float*)0x2000;
  EXPECT(kvq_decode_attention(&k, (void*)0x1000, 299, out, (void*)0x3000, ws, 0, nullptr) == KVQ_EHIP);
  EXPECT(kvq_decode_attention(&k, (void*)0x1000, 299, out, (void*)0x3000, ws - 1, 0, nullptr) == KVQ_EWORKSPACE);
  EXPECT(kvq_decode_attention(&k, (void*)0x1000, -1, out, (void*)0x3000, ws, 0, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_decode_attention(&k, (void*)0x1000, 299, out, (void*)0x3000, ws, 4097, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_decode_attention(&k, nullptr, 299, out, (void*)0x3000, ws, 0, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_decode_attention_noalloc(&k, (void*)0x1000, 299, out, 0, nullptr) != KVQ_OK);   // no GPU here
  EXPECT(kvq_decode_attention_noalloc(&k, (void*)0x1000, 299, out, -3, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_decode_attention_noalloc(&k, nullptr, 299, out, 0, nullptr) == KVQ_EINVAL);
  kvq_config big = base();
  big.batch = 8; big.q_heads = 32; big.kv_heads = 32;
  kvq_cache kb = fake_cache(big, 100);
  EXPECT(kvq_decode_attention_noalloc(&kb, (void*)0x1000, 99, out, 4096, nullptr) == KVQ_EWORKSPACE);
  // chunk of queries: workspace sizing and argument checks
  EXPECT(kvq_chunk_workspace_bytes(&k, 5, 3) == (size_t)2 * 8 * 5 * 3 * 130 * 4);
  EXPECT(kvq_chunk_workspace_bytes(&k, 0, 3) == 0 && kvq_chunk_workspace_bytes(&k, 1025, 3) == 0);
  EXPECT(kvq_chunk_workspace_bytes(&k, 5, -1) == 0 && kvq_chunk_workspace_bytes(nullptr, 5, 3) == 0);
  const size_t cws = kvq_chunk_workspace_bytes(&k, 5, 0);
  EXPECT(cws > 0 && cws % ((size_t)2 * 8 * 5 * 130 * 4) == 0);
  EXPECT(kvq_chunk_attention(&k, (void*)0x1000, 5, 295, out, (void*)0x3000, cws, 0, nullptr) == KVQ_EHIP);
  EXPECT(kvq_chunk_attention(&k, (void*)0x1000, 5, 295, out, (void*)0x3000, cws - 1, 0, nullptr) == KVQ_EWORKSPACE);
  EXPECT(kvq_chunk_attention(&k, (void*)0x1000, 0, 295, out, (void*)0x3000, cws, 0, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_chunk_attention(&k, (void*)0x1000, 1025, 0, out, (void*)0x3000, cws, 0, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_chunk_attention(&k, (void*)0x1000, 5, -1, out, (void*)0x3000, cws, 0, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_chunk_attention(&k, (void*)0x1000, 5, 295, out, (void*)0x3000, cws, 4097, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_chunk_attention(&k, nullptr, 5, 295, out, (void*)0x3000, cws, 0, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_chunk_attention(&k, (void*)0x1000, 5, 295, nullptr, (void*)0x3000, cws, 0, nullptr) == KVQ_EINVAL);
  // fused decode step: argument checks, workspace, capacity, then the (stubbed) launch
  EXPECT(kvq_decode_step(&k, (void*)0x1000, (void*)0x1000, (void*)0x1000, out, (void*)0x3000, ws, 0, nullptr) ==
         KVQ_EHIP);
  EXPECT(k.length == 300);
  EXPECT(kvq_decode_step(&k, (void*)0x1000, (void*)0x1000, (void*)0x1000, out, (void*)0x3000, ws, 3, nullptr) ==
         KVQ_EHIP);
  EXPECT(kvq_decode_step(&k, (void*)0x1000, (void*)0x1000, (void*)0x1000, out, (void*)0x3000, ws - 1, 0, nullptr) ==
         KVQ_EWORKSPACE);
  EXPECT(kvq_decode_step(&k, (void*)0x1000, (void*)0x1000, (void*)0x1000, out, nullptr, ws, 0, nullptr) ==
         KVQ_EWORKSPACE);
  EXPECT(kvq_decode_step(&k, (void*)0x1000, (void*)0x1000, (void*)0x1000, out, (void*)0x3000, ws, -1, nullptr) ==
         KVQ_EINVAL);
  EXPECT(kvq_decode_step(&k, (void*)0x1000, (void*)0x1000, (void*)0x1000, out, (void*)0x3000, ws, 4097, nullptr) ==
         KVQ_EINVAL);
  EXPECT(kvq_decode_step(&k, nullptr, (void*)0x1000, (void*)0x1000, out, (void*)0x3000, ws, 0, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_decode_step(&k, (void*)0x1000, (void*)0x1000, (void*)0x1000, nullptr, (void*)0x3000, ws, 0, nullptr) ==
         KVQ_EINVAL);
  EXPECT(k.length == 300);
  k.length = 1024;
  EXPECT(kvq_decode_step(&k, (void*)0x1000, (void*)0x1000, (void*)0x1000, out, (void*)0x3000, ws, 0, nullptr) ==
         KVQ_ECAPACITY);
  k.length = 300;
  EXPECT(kvq_dequantize(&k, 0, 0, 300, out, nullptr) == KVQ_EHIP);
  EXPECT(kvq_dequantize(&k, 2, 0, 300, out, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_dequantize(&k, 1, 10, 5, out, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_dequantize(&k, 1, 0, 301, out, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_dequantize(&k, 1, 7, 7, nullptr, nullptr) == KVQ_OK);
  k.v_scale = nullptr;
  EXPECT(kvq_quantize_append(&k, (void*)0x1000, (void*)0x1000, 5, nullptr) == KVQ_EINVAL);
  EXPECT(kvq_decode_attention(&k, (void*)0x1000, 299, out, (void*)0x3000, ws, 0, nullptr) == KVQ_EINVAL);
  // paged layout and per-sequence lengths: sizes, descriptor checks, what each call
  // accepts; the host lengths change only when every launch succeeded
  {
    kvq_config c = base();
    kvq_layout dense, paged;
    EXPECT(kvq_cache_layout(&c, &dense) == KVQ_OK);
    EXPECT(kvq_paged_layout(&c, 5, &paged) == KVQ_OK);
    const size_t dslots = (size_t)2 * 2 * 8, pslots = (size_t)5 * 2;  // batch*kv_heads*T/Bk, pool*kv_heads
    EXPECT(paged.k_codes == dense.k_codes / dslots * pslots && paged.v_scale == dense.v_scale / dslots * pslots);
    EXPECT(paged.k_col == dense.k_col / dslots * pslots && paged.k_scale == dense.k_scale / dslots * pslots);
    EXPECT(paged.k_rowptr == pslots * 129 * 4 && paged.k_tail == dense.k_tail && paged.rope == dense.rope);
    EXPECT(kvq_paged_layout(&c, 0, &paged) == KVQ_EINVAL && kvq_paged_layout(&c, 1 << 30, &paged) == KVQ_EINVAL);
    kvq_cache p = fake_cache(c, 0);
    int64_t host[2] = {300, 0};
    p.seq_lens_host = host;
    EXPECT(kvq_cache_init(&p, nullptr) == KVQ_EINVAL);           // host lengths without device ones
    p.seq_lens = (int64_t*)0x5000;
    p.block_table = (const int32_t*)0x6000;
    EXPECT(kvq_cache_init(&p, nullptr) == KVQ_EINVAL);           // a table without a pool size
    p.num_blocks = 5;
    EXPECT(kvq_cache_init(&p, nullptr) == KVQ_EHIP);
    EXPECT(host[0] == 300);
    host[1] = 2000;
    EXPECT(kvq_quantize_append(&p, (void*)0x1000, (void*)0x1000, 1, nullptr) == KVQ_EINVAL);  // length > T
    host[1] = 1000;
    EXPECT(kvq_quantize_append(&p, (void*)0x1000, (void*)0x1000, 30, nullptr) == KVQ_ECAPACITY);
    EXPECT(kvq_quantize_append(&p, (void*)0x1000, (void*)0x1000, 20, nullptr) == KVQ_EHIP);
    EXPECT(host[0] == 300 && host[1] == 1000);
    const size_t pws = kvq_decode_workspace_bytes(&p, 0);
    EXPECT(kvq_decode_attention(&p, (void*)0x1000, -1, out, (void*)0x3000, pws, 0, nullptr) == KVQ_EHIP);
    EXPECT(kvq_decode_attention(&p, (void*)0x1000, 299, out, (void*)0x3000, pws, 0, nullptr) == KVQ_EINVAL);
    EXPECT(kvq_decode_attention_noalloc(&p, (void*)0x1000, -1, out, 0, nullptr) == KVQ_EHIP);
    host[1] = 0;
    EXPECT(kvq_decode_attention(&p, (void*)0x1000, -1, out, (void*)0x3000, pws, 0, nullptr) == KVQ_EINVAL);
    EXPECT(kvq_chunk_attention(&p, (void*)0x1000, 4, 0, out, (void*)0x3000, 1 << 30, 0, nullptr) ==
           KVQ_EUNSUPPORTED);
    EXPECT(kvq_decode_step(&p, (void*)0x1000, (void*)0x1000, (void*)0x1000, out, (void*)0x3000, pws, 0, nullptr) ==
           KVQ_EUNSUPPORTED);
    EXPECT(kvq_dequantize(&p, 0, 0, 1, out, nullptr) == KVQ_EUNSUPPORTED);
    // ragged append: counts in [0, n_max], capacity per sequence, nothing to do
    host[0] = 300; host[1] = 1000;
    const int64_t cnt_ok[2] = {5, 24}, cnt_cap[2] = {5, 25}, cnt_bad[2] = {-1, 3}, cnt_zero[2] = {0, 0};
    const int64_t* dev_cnt = (const int64_t*)0x7000;
    EXPECT(kvq_quantize_append_seqs(&p, (void*)0x1000, (void*)0x1000, 24, cnt_ok, dev_cnt, nullptr) == KVQ_EHIP);
    EXPECT(kvq_quantize_append_seqs(&p, (void*)0x1000, (void*)0x1000, 30, cnt_cap, dev_cnt, nullptr) ==
           KVQ_ECAPACITY);
    EXPECT(kvq_quantize_append_seqs(&p, (void*)0x1000, (void*)0x1000, 23, cnt_ok, dev_cnt, nullptr) == KVQ_EINVAL);
    EXPECT(kvq_quantize_append_seqs(&p, (void*)0x1000, (void*)0x1000, 24, cnt_bad, dev_cnt, nullptr) == KVQ_EINVAL);
    EXPECT(kvq_quantize_append_seqs(&p, (void*)0x1000, (void*)0x1000, 24, cnt_ok, nullptr, nullptr) == KVQ_EINVAL);
    EXPECT(kvq_quantize_append_seqs(&p, nullptr, nullptr, 24, cnt_zero, dev_cnt, nullptr) == KVQ_OK);
    EXPECT(kvq_quantize_append_seqs(&p, nullptr, (void*)0x1000, 24, cnt_ok, dev_cnt, nullptr) == KVQ_EINVAL);
    EXPECT(host[0] == 300 && host[1] == 1000);
    p.block_table = nullptr;  // per-sequence lengths over the dense slots
    host[1] = 7;
    EXPECT(kvq_quantize_append(&p, (void*)0x1000, (void*)0x1000, 3, nullptr) == KVQ_EHIP);
    EXPECT(kvq_decode_attention(&p, (void*)0x1000, -1, out, (void*)0x3000, pws, 0, nullptr) == KVQ_EHIP);
    p.seq_lens = nullptr;
    EXPECT(kvq_quantize_append(&p, (void*)0x1000, (void*)0x1000, 3, nullptr) == KVQ_EINVAL);  // one copy only
    kvq_cache dcache = fake_cache(base(), 100);
    EXPECT(kvq_quantize_append_seqs(&dcache, (void*)0x1000, (void*)0x1000, 24, cnt_ok, dev_cnt, nullptr) ==
           KVQ_EINVAL);
  }
  printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
