// dequantize.hip -- packed cache -> fp32 values (pre-RoPE).
//
// x = fmaf(code, scale, zero) with one fp32 rounding, or the codebook entry for
// codebook keys; outlier positions take their exact fp16 value from the CSR, kept keys
// their fp16 rows, and the tail tokens are exact.  This is the read-side inverse of the per-block scale and
// zero-point storage of "【LLM量化技术介绍-3】KV Cache量化技术介绍"
// (developer.horizon.auto/blog/13163), section "Quanto 的量化原理".
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

// One thread per (token, channel); grid.y = b * kv_heads + h.
__global__ void dequantize_kernel(kvq_cache c, int which, int64_t t0, int64_t t1,
                                  float* __restrict__ out) {
  const int D = c.cfg.head_dim, Bk = c.cfg.k_block;
  const int64_t T = c.cfg.capacity;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % c.cfg.kv_heads);
  const int64_t nfull = (c.length / Bk) * Bk;
  const int ko = kout_of(c.cfg);
  const int64_t total = (t1 - t0) * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = t0 + i / D;
    const int ch = (int)(i % D);
    float x;
    if (t >= nfull) {
      const uint16_t* tail = which ? c.v_tail : c.k_tail;
      x = h2f(tail[(bh * Bk + (t - nfull)) * D + ch]);
    } else if (which == 0) {
      const int kb = c.cfg.k_bits;
      const int e = ch < D / 2 ? 2 * ch : 2 * (ch - D / 2) + 1;  // element holding channel ch
      const uint8_t* row = static_cast<const uint8_t*>(c.k_codes) + (bh * T + t) * (D * kb / 8);
      const int pos = e * kb;
      uint32_t w = row[pos >> 3];
      if ((pos & 7) + kb > 8) w |= (uint32_t)row[(pos >> 3) + 1] << 8;
      const uint32_t code = (w >> (pos & 7)) & ((1u << kb) - 1u);
      if (c.cfg.k_mode == 2) {
        x = e4m3_to_f32(code);
      } else if (c.cfg.k_mode == 1) {
        x = h2f(c.k_lut[((int64_t)h * D + ch) * (1 << kb) + code]);
      } else {
        const int64_t m = (bh * (T / Bk) + t / Bk) * D + ch;
        x = __builtin_fmaf((float)code, h2f(c.k_scale[m]), h2f(c.k_zero[m]));
      }
    } else {
      const int vb = c.cfg.v_bits, tpw = 32 / vb, G = c.cfg.v_group;
      const uint32_t* words = static_cast<const uint32_t*>(c.v_codes) + bh * (T / tpw) * D;
      const uint32_t code = (words[(t / tpw) * D + ch] >> ((t % tpw) * vb)) & ((1u << vb) - 1u);
      if (c.cfg.v_mode == 2) {
        x = e4m3_to_f32(code);
      } else if (c.cfg.v_mode == 1) {
        x = h2f(c.v_lut[((int64_t)h * D + ch) * (1 << vb) + code]);
      } else {
        const int64_t m = (bh * T + t) * (D / G) + ch / G;
        x = __builtin_fmaf((float)code, h2f(c.v_scale[m]), h2f(c.v_zero[m]));
      }
    }
    if (t < nfull && ko > 0) {
      const uint8_t* col = which ? c.v_col : c.k_col;
      const uint16_t* val = which ? c.v_val : c.k_val;
      for (int r = 0; r < ko; ++r)
        if (col[(bh * T + t) * ko + r] == ch) x = h2f(val[(bh * T + t) * ko + r]);
    }
    const int R = keep_count(c.cfg);
    if (t < nfull && which == 0 && R > 0) {  // a key kept in fp16 reads back exactly
      const int64_t slot = bh * (T / Bk) + t / Bk;
      for (int r = 0; r < R; ++r)
        if (c.k_keep_idx[slot * R + r] == (uint8_t)(t % Bk)) x = h2f(c.k_keep_val[(slot * R + r) * D + ch]);
    }
    out[bh * (t1 - t0) * D + i] = x;
  }
}

}  // namespace

hipError_t launch_dequantize(const kvq_cache& c, int which, int64_t t0, int64_t t1, float* out,
                             hipStream_t s) {
  const int64_t BH = (int64_t)c.cfg.batch * c.cfg.kv_heads;
  if (BH > 65535) return hipErrorInvalidValue;
  const int64_t work = (t1 - t0) * c.cfg.head_dim;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)blocks, (unsigned)BH), dim3(256), 0, s, c,
                     which, t0, t1, out);
  return hipGetLastError();
}

}  // namespace kvq
