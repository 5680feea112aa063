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

// Four fp16 values (bits) to E4M3 bytes 0..3 of a word.  The hardware conversion rounds
// to nearest even and, with the inputs clamped to +-448 first (med3), equals the
// saturating cast f16_to_e4m3 for every non-NaN input (checked on all 65536); a word
// with a NaN input (the clamp would lose it) takes the integer cast.
__device__ __forceinline__ uint32_t e4m3x4(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3) {
  const float x0 = h2f((uint16_t)h0), x1 = h2f((uint16_t)h1), x2 = h2f((uint16_t)h2), x3 = h2f((uint16_t)h3);
  if (__builtin_expect(x0 != x0 || x1 != x1 || x2 != x2 || x3 != x3, 0))
    return f16_to_e4m3(h0) | (f16_to_e4m3(h1) << 8) | (f16_to_e4m3(h2) << 16) | (f16_to_e4m3(h3) << 24);
  const float c0 = __builtin_amdgcn_fmed3f(x0, -448.0f, 448.0f), c1 = __builtin_amdgcn_fmed3f(x1, -448.0f, 448.0f);
  const float c2 = __builtin_amdgcn_fmed3f(x2, -448.0f, 448.0f), c3 = __builtin_amdgcn_fmed3f(x3, -448.0f, 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, lo, true);
}

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
    for (int w = 0; w < 4; ++w)  // pairs i0 + 2w, i0 + 2w + 1: bytes a, b, a, b
      out[w] = e4m3x4(a[w] & 0xFFFFu, bb[w] & 0xFFFFu, a[w] >> 16, bb[w] >> 16);
    *reinterpret_cast<uint4*>(krow + (int64_t)j * D + 2 * i0) = make_uint4(out[0], out[1], out[2], out[3]);
  }
  // values
  uint32_t* vwords = static_cast<uint32_t*>(c.v_codes) + g * (BK / 4) * D;
  for (int task = threadIdx.x; task < (BK / 4) * (D / 8); task += kThreads) {
    const int tg = task / (D / 8), c0 = 8 * (task % (D / 8));
    uint32_t x[4][4];  // [token u][dword]: channels c0 .. c0 + 7 of the group's 4 tokens
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t* row = src_row(c.v_tail, v_new, bh, BK, D, t0 + 4 * tg + u, tail0, old_len, n_new);
      const uint4 x4 = *reinterpret_cast<const uint4*>(row + c0);
      x[u][0] = x4.x; x[u][1] = x4.y; x[u][2] = x4.z; x[u][3] = x4.w;
    }
    uint32_t wd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // channel c0 + e: its 4 tokens' bytes
      const int dw = e >> 1, sh = 16 * (e & 1);
      wd[e] = e4m3x4((x[0][dw] >> sh) & 0xFFFFu, (x[1][dw] >> sh) & 0xFFFFu, (x[2][dw] >> sh) & 0xFFFFu,
                     (x[3][dw] >> sh) & 0xFFFFu);
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
