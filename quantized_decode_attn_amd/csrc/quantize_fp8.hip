// quantize_fp8.hip -- the FP8 cache: keys and values of a completed block cast to OCP
// E4M3, one byte per element, no statistics ([UQ] section 2.1: an FP8 cache halves the
// fp16 cache, its exponent bits keeping the dynamic range).
//
// Pages cited (title, address):
//   [UQ] "大模型长上下文推理优化：4-bit KV Cache量化技术解析与部署实践", mlqm.cn/news/1064729
//   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

// Token t of the block's (b, h): from the tail (t < old_len) or from the new rows.
__device__ __forceinline__ const uint16_t* src_row(const uint16_t* tail, const uint16_t* src_new, int64_t bh, int BK,
                                                   int D, int64_t t, int64_t tail0, int64_t old_len, int64_t n_new) {
  return t < old_len ? tail + (bh * BK + (t - tail0)) * D : src_new + (bh * n_new + (t - old_len)) * D;
}

// One block of (b, h) per workgroup.  Keys keep the packed key row order (element e
// holds channel (e >> 1) + (e & 1) D/2, [KVC3] "Pre-RoPE Key Quantization" pairs): a
// task reads 8 channels of each rotary half of one token and writes 16 row bytes.
// Values keep the value word order (a word holds 4 consecutive tokens of one channel):
// a task reads 8 channels of 4 tokens and writes 8 words.
template <int D, int BK>
__global__ __launch_bounds__(kThreads) void quantize_fp8_kernel(kvq_cache c, const uint16_t* __restrict__ k_new,
                                                                const uint16_t* __restrict__ v_new, int64_t old_len_arg,
                                                                int64_t n_new, int64_t n_first,
                                                                const int64_t* __restrict__ n_seq) {
  constexpr int HALF = D / 2;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t old_len = c.seq_lens ? seq_len_of(c, b) : old_len_arg;
  const int64_t n_b = n_seq ? min(max(n_seq[b], (int64_t)0), n_new) : n_new;
  const int64_t n = (c.seq_lens ? old_len / BK : n_first) + blockIdx.x;
  if (n >= (old_len + n_b) / BK || n >= c.cfg.capacity / BK) return;
  const int64_t g = slot_of(c, b, h, n);
  const int64_t bh = (int64_t)b * c.cfg.kv_heads + h;
  const int64_t t0 = n * BK, tail0 = (old_len / BK) * BK;
  // keys
  uint8_t* krow = static_cast<uint8_t*>(c.k_codes) + g * BK * D;
  for (int task = threadIdx.x; task < BK * (HALF / 8); task += kThreads) {
    const int j = task / (HALF / 8), i0 = 8 * (task % (HALF / 8));
    const uint16_t* row = src_row(c.k_tail, k_new, bh, BK, D, t0 + j, tail0, old_len, n_new);
    const uint4 a4 = *reinterpret_cast<const uint4*>(row + i0);
    const uint4 b4 = *reinterpret_cast<const uint4*>(row + HALF + i0);
    const uint32_t a[4] = {a4.x, a4.y, a4.z, a4.w}, bb[4] = {b4.x, b4.y, b4.z, b4.w};
    uint32_t out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // pairs i0 + 2w, i0 + 2w + 1: bytes a, b, a, b
      out[w] = f16_to_e4m3(a[w] & 0xFFFFu) | (f16_to_e4m3(bb[w] & 0xFFFFu) << 8) |
               (f16_to_e4m3(a[w] >> 16) << 16) | (f16_to_e4m3(bb[w] >> 16) << 24);
    }
    *reinterpret_cast<uint4*>(krow + (int64_t)j * D + 2 * i0) = make_uint4(out[0], out[1], out[2], out[3]);
  }
  // values
  uint32_t* vwords = static_cast<uint32_t*>(c.v_codes) + g * (BK / 4) * D;
  for (int task = threadIdx.x; task < (BK / 4) * (D / 8); task += kThreads) {
    const int tg = task / (D / 8), c0 = 8 * (task % (D / 8));
    uint32_t wd[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t* row = src_row(c.v_tail, v_new, bh, BK, D, t0 + 4 * tg + u, tail0, old_len, n_new);
      const uint4 x4 = *reinterpret_cast<const uint4*>(row + c0);
      const uint32_t x[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) wd[e] |= f16_to_e4m3((x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << (8 * u);
    }
    *reinterpret_cast<uint4*>(vwords + (int64_t)tg * D + c0) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    *reinterpret_cast<uint4*>(vwords + (int64_t)tg * D + c0 + 4) = make_uint4(wd[4], wd[5], wd[6], wd[7]);
  }
}

template <int D, int BK>
hipError_t launch_fp8(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new, int64_t old_len,
                      int64_t n_new, int64_t n_first, int64_t nblocks, const int64_t* n_seq, hipStream_t s) {
  dim3 grid((unsigned)nblocks, (unsigned)c.cfg.kv_heads, (unsigned)c.cfg.batch);
  hipLaunchKernelGGL((quantize_fp8_kernel<D, BK>), grid, dim3(kThreads), 0, s, c, k_new, v_new, old_len, n_new,
                     n_first, n_seq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fp8(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new, int64_t old_len,
                               int64_t n_new, int64_t n_first, int64_t nblocks, const int64_t* n_seq,
                               hipStream_t s) {
  const int D = c.cfg.head_dim, Bk = c.cfg.k_block;
  if (D == 128 && Bk == 128) return launch_fp8<128, 128>(c, k_new, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 128 && Bk == 64) return launch_fp8<128, 64>(c, k_new, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 64 && Bk == 128) return launch_fp8<64, 128>(c, k_new, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (D == 64 && Bk == 64) return launch_fp8<64, 64>(c, k_new, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
