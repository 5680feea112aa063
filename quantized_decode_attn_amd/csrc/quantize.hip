// quantize.hip -- append-time quantization of complete token blocks, tail copy and
// the rotary tables.
//
// Pages cited (title, address):
//   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
//   [UQ]   "大模型长上下文推理优化：4-bit KV Cache量化技术解析与部署实践", mlqm.cn/news/1064729
//   [TQ]   "TurboQuant：突破大模型推理瓶颈的KVCache量化技术解析", mlqm.cn/news/1002276
//
// One workgroup (256 threads, 4 waves) owns one (b, kv-head, block, tensor): the
// k_block x head_dim fp16 tile is staged once in LDS and every step below reads it
// from there.  The steps, in the order the pages give them:
//   1. dense-and-sparse split: per token vector, the ko largest |x| go to the CSR
//      ([KVC3] "Per-Vector Dense-and-Sparse Quantization");
//   2. clip threshold: exact q-quantile of |x| over the tile by radix selection on the
//      15-bit fp16 magnitudes, linear interpolation in fp64 ([UQ] section 4.2);
//   3. statistics: keys per channel over the block ([KVC3] "Per-Channel Key
//      Quantization", before RoPE per "Pre-RoPE Key Quantization"), values per token
//      over channel groups ([KVC3] "Quanto 的量化原理"); fp16 zero rounded down and
//      fp16 scale rounded up;
//   4. codes: round-half-even((d - zero) / scale) with IEEE fp32 subtract and divide
//      (round(x/scale) of [TQ] section 4.2), or nearest codebook entry
//      ([KVC3] "Non-Uniform KV Cache Quantization"); outlier positions get code 0;
//   5. packing and 128-bit stores.
// Every floating-point operation whose result decides a stored bit is a single IEEE
// fp32 (or, for the quantile interpolation, fp64) operation, built without FMA
// contraction, so that the stored caches are reproducible bit for bit.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- rotary tables
__global__ void rope_init_kernel(float* rope, int D, int Bk, int nblk, float theta) {
  const int half = D / 2;
  const int64_t total = (int64_t)(Bk + nblk) * half;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx % half);
    const int64_t row = idx / half;
    const double pos = row < Bk ? (double)row : (double)(row - Bk) * (double)Bk;
    const double f = pow((double)theta, -(2.0 * i) / (double)D);
    double sn, cs;
    sincos(pos * f, &sn, &cs);
    rope[2 * idx] = (float)cs;
    rope[2 * idx + 1] = (float)sn;
  }
}

// ---------------------------------------------------------------- block reductions
struct Red {
  float f[kThreads / kWave];
  uint32_t u[kThreads / kWave];
  int32_t i[kThreads / kWave];
};

__device__ uint32_t block_sum_u32(uint32_t v, Red& r) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.u[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) s += r.u[w];
  return s;
}
__device__ uint32_t block_min_u32(uint32_t v, Red& r) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m, kWave));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.u[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t s = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) s = min(s, r.u[w]);
  return s;
}

// First bin where the running count exceeds `rank`; returns the bin and the count
// of everything below it.  Wave 0 scans, the result is broadcast through LDS.
__device__ void find_bin(const uint32_t* hist, int nbins, uint32_t rank, int* out_bin,
                         uint32_t* out_below, int* sh_bin, uint32_t* sh_below) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = nbins / kWave;
    uint32_t local = 0;
    for (int k = 0; k < per; ++k) local += hist[lane * per + k];
    uint32_t incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      uint32_t o = (uint32_t)__shfl_up((int)incl, d, kWave);
      if (lane >= d) incl += o;
    }
    const uint64_t over = __ballot(incl > rank);
    const int first = __ffsll((unsigned long long)over) - 1;
    if (lane == first) {
      uint32_t below = incl - local;
      int b = lane * per;
      for (int k = 0; k < per; ++k) {
        const uint32_t h = hist[lane * per + k];
        if (below + h > rank) { b = lane * per + k; break; }
        below += h;
      }
      *sh_bin = b;
      *sh_below = below;
    }
  }
  __syncthreads();
  *out_bin = *sh_bin;
  *out_below = *sh_below;
}

// ---------------------------------------------------------------- the block kernel
template <int D, int BK>
struct QShared {
  static constexpr int kPitch = D + 8;  // halves per LDS row (16-byte padding)
  uint16_t tile[BK * kPitch];
  uint32_t mask[BK * (D / 32)];
  float meta_z[BK * (D / 16) > D ? BK * (D / 16) : D];
  float meta_s[BK * (D / 16) > D ? BK * (D / 16) : D];
  float mids[D * 15];
  float part_lo[kThreads], part_hi[kThreads];
  int part_n[kThreads];
  uint32_t hist[256];
  Red red;
  int sh_bin;
  uint32_t sh_below;
  float thr;
};

__device__ __forceinline__ int code_uniform(float d, float z, float s, int L) {
  if (s == 0.0f) return 0;
  const float num = d - z;
  const float q = num / s;  // IEEE-correct fp32 division
  float r = __builtin_rintf(q);
  r = fmaxf(r, 0.0f);
  r = fminf(r, (float)L);
  return (int)r;
}

__device__ __forceinline__ void meta_from(float lo, float hi, int cnt, int L, uint16_t* z16,
                                          uint16_t* s16) {
  if (cnt == 0) { lo = 0.0f; hi = 0.0f; }
  lo = lo + 0.0f;
  hi = hi + 0.0f;
  *z16 = f2h_rd(lo);
  const float range = hi - h2f(*z16);
  const float s32 = range / (float)L;
  *s16 = f2h_ru(s32);
}

// Key rows: 32 elements (16 rotary pairs: channels m and m + D/2) per work item,
// packed LSB first into KB dwords and written with one vector store.
template <int D, int BK, int KB, typename CodeFn>
__device__ __forceinline__ void pack_key_rows(uint8_t* out, CodeFn code_of) {
  constexpr int kChunksPerRow = D / 32;
  constexpr int kRowBytes = D * KB / 8;
  for (int idx = threadIdx.x; idx < BK * kChunksPerRow; idx += kThreads) {
    const int j = idx / kChunksPerRow, cch = idx % kChunksPerRow;
    uint32_t w[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) w[k] = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int ch = cch * 16 + (e >> 1) + (e & 1) * (D / 2);
      const uint32_t code = code_of(j, ch);
      const int pos = e * KB;
      w[pos >> 5] |= code << (pos & 31);
      if ((pos & 31) + KB > 32) w[(pos >> 5) + 1] |= code >> (32 - (pos & 31));
    }
    uint8_t* dst = out + (int64_t)j * kRowBytes + cch * 4 * KB;
    if constexpr (KB == 4) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (KB == 2) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int k = 0; k < KB; ++k) reinterpret_cast<uint32_t*>(dst)[k] = w[k];
    }
  }
}

template <int D, int BK>
__global__ __launch_bounds__(kThreads) void quantize_blocks_kernel(
    kvq_cache c, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    int64_t old_len, int64_t n_new, int64_t n_first) {
  __shared__ QShared<D, BK> sh;
  constexpr int P = QShared<D, BK>::kPitch;
  const int tid = threadIdx.x;
  const int is_key = (blockIdx.x & 1) == 0;
  const int64_t n = n_first + (blockIdx.x >> 1);
  const int h = blockIdx.y, b = blockIdx.z;
  const int H = c.cfg.kv_heads;
  const int64_t T = c.cfg.capacity;
  const int64_t bh = (int64_t)b * H + h;
  const int bits = is_key ? c.cfg.k_bits : c.cfg.v_bits;
  const int L = (1 << bits) - 1;
  const int ko = kout_of(c.cfg);
  const int64_t t0 = n * BK;
  const int64_t nf_old = old_len / BK;

  // 1. stage the tile (rows from the old tail or from the new input)
  {
    const uint16_t* tail = is_key ? c.k_tail : c.v_tail;
    const uint16_t* src_new = is_key ? k_new : v_new;
    constexpr int kChunks = BK * D / 8;
    for (int idx = tid; idx < kChunks; idx += kThreads) {
      const int j = idx / (D / 8), part = idx % (D / 8);
      const int64_t t = t0 + j;
      const uint16_t* row = t < old_len ? tail + (bh * BK + (t - nf_old * BK)) * D
                                        : src_new + (bh * n_new + (t - old_len)) * D;
      const uint4 v = *reinterpret_cast<const uint4*>(row + part * 8);
      *reinterpret_cast<uint4*>(&sh.tile[j * P + part * 8]) = v;
    }
    for (int idx = tid; idx < BK * (D / 32); idx += kThreads) sh.mask[idx] = 0;
  }
  __syncthreads();

  // 2. dense-and-sparse split: 16 lanes per token row
  if (ko > 0) {
    int32_t* rowptr = is_key ? c.k_rowptr : c.v_rowptr;
    uint8_t* col_out = is_key ? c.k_col : c.v_col;
    uint16_t* val_out = is_key ? c.k_val : c.v_val;
    const int lane = tid & 63, wave = tid >> 6;
    const int sub = lane & 15;
    constexpr int kPer = D / 16;
    for (int pass = 0; pass < BK / 16; ++pass) {
      const int j = pass * 16 + wave * 4 + (lane >> 4);
      uint32_t top[4] = {0, 0, 0, 0};  // keys: (|x| bits << 8) | (255 - col), descending
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int col = sub * kPer + k;
        uint32_t key = ((uint32_t)(sh.tile[j * P + col] & 0x7fff) << 8) | (uint32_t)(255 - col);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t hi = max(top[r], key), lo = min(top[r], key);
          top[r] = hi;
          key = lo;
        }
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        uint32_t other[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) other[r] = (uint32_t)__shfl_xor((int)top[r], m, kWave);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint32_t key = other[r];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint32_t hi = max(top[s], key), lo = min(top[s], key);
            top[s] = hi;
            key = lo;
          }
        }
      }
      if (sub == 0) {
        int cols[4];
        for (int r = 0; r < ko; ++r) cols[r] = 255 - (int)(top[r] & 0xff);
        for (int a = 1; a < ko; ++a)
          for (int q = a; q > 0 && cols[q - 1] > cols[q]; --q) {
            const int t = cols[q]; cols[q] = cols[q - 1]; cols[q - 1] = t;
          }
        const int64_t t = t0 + j;
        uint32_t words[D / 32];
        for (int w = 0; w < D / 32; ++w) words[w] = 0;
        for (int r = 0; r < ko; ++r) {
          col_out[(bh * T + t) * ko + r] = (uint8_t)cols[r];
          val_out[(bh * T + t) * ko + r] = sh.tile[j * P + cols[r]];
          words[cols[r] >> 5] |= 1u << (cols[r] & 31);
        }
        for (int w = 0; w < D / 32; ++w) sh.mask[j * (D / 32) + w] = words[w];
        rowptr[bh * (T + 1) + t + 1] = (int32_t)((t + 1) * ko);
        if (t == 0) rowptr[bh * (T + 1)] = 0;
      }
    }
  }

  // 3. clip threshold: exact order statistics of |x| over the whole tile
  const bool clip = c.cfg.clip_quantile > 0.0f;
  if (clip) {
    constexpr int NEL = BK * D;
    const double pos = (double)c.cfg.clip_quantile * (double)(NEL - 1);
    const int64_t kr = (int64_t)floor(pos);
    const double frac = pos - (double)kr;
    // pass 1: top 8 of the 15 magnitude bits
    for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < NEL; i += kThreads) {
      const uint32_t key = sh.tile[(i / D) * P + (i % D)] & 0x7fff;
      atomicAdd(&sh.hist[key >> 7], 1u);
    }
    __syncthreads();
    int bin1;
    uint32_t below1;
    find_bin(sh.hist, 256, (uint32_t)kr, &bin1, &below1, &sh.sh_bin, &sh.sh_below);
    __syncthreads();
    // pass 2: low 7 bits inside the selected bin
    for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < NEL; i += kThreads) {
      const uint32_t key = sh.tile[(i / D) * P + (i % D)] & 0x7fff;
      if ((int)(key >> 7) == bin1) atomicAdd(&sh.hist[key & 127], 1u);
    }
    __syncthreads();
    int bin2;
    uint32_t below2;
    find_bin(sh.hist, 128, (uint32_t)kr - below1, &bin2, &below2, &sh.sh_bin, &sh.sh_below);
    const uint32_t vk = ((uint32_t)bin1 << 7) | (uint32_t)bin2;
    // the next order statistic: equal to vk if vk repeats past rank kr, else the
    // smallest magnitude above vk
    uint32_t le = 0, gt_min = 0xffffffffu;
    for (int i = tid; i < NEL; i += kThreads) {
      const uint32_t key = sh.tile[(i / D) * P + (i % D)] & 0x7fff;
      le += key <= vk;
      if (key > vk) gt_min = min(gt_min, key);
    }
    le = block_sum_u32(le, sh.red);
    gt_min = block_min_u32(gt_min, sh.red);
    if (tid == 0) {
      float t;
      const double v0 = (double)h2f((uint16_t)vk);
      if (kr + 1 >= NEL) {
        t = (float)v0;
      } else {
        const uint32_t vk1 = le >= (uint32_t)(kr + 2) ? vk : gt_min;
        const double v1 = (double)h2f((uint16_t)vk1);
        const double diff = v1 - v0;
        const double prod = frac * diff;
        const double sum = v0 + prod;
        t = (float)sum;
      }
      sh.thr = t;
    }
  }
  __syncthreads();
  const float thr = clip ? sh.thr : 0.0f;

  auto dense = [&](int j, int ch) -> float {
    const float x = h2f(sh.tile[j * P + ch]);
    return clip ? fminf(fmaxf(x, -thr), thr) : x;
  };
  auto is_out = [&](int j, int ch) -> bool {
    return (sh.mask[j * (D / 32) + (ch >> 5)] >> (ch & 31)) & 1u;
  };

  // 4. statistics and metadata
  if (is_key && c.cfg.k_mode == 1) {
    for (int ch = tid; ch < D; ch += kThreads) {
      const uint16_t* lut = c.k_lut + ((int64_t)h * D + ch) * (L + 1);
      for (int k = 0; k < L; ++k) sh.mids[ch * 15 + k] = (h2f(lut[k]) + h2f(lut[k + 1])) * 0.5f;
    }
  } else if (is_key) {
    constexpr int kParts = kThreads / D;
    const int ch = tid % D, part = tid / D;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    int cnt = 0;
    for (int j = part; j < BK; j += kParts) {
      if (is_out(j, ch)) continue;
      const float d = dense(j, ch);
      lo = fminf(lo, d);
      hi = fmaxf(hi, d);
      ++cnt;
    }
    sh.part_lo[tid] = lo;
    sh.part_hi[tid] = hi;
    sh.part_n[tid] = cnt;
    __syncthreads();
    if (part == 0) {
      for (int p = 1; p < kParts; ++p) {
        lo = fminf(lo, sh.part_lo[tid + p * D]);
        hi = fmaxf(hi, sh.part_hi[tid + p * D]);
        cnt += sh.part_n[tid + p * D];
      }
      uint16_t z16, s16;
      meta_from(lo, hi, cnt, L, &z16, &s16);
      c.k_scale[(bh * (T / BK) + n) * D + ch] = s16;
      c.k_zero[(bh * (T / BK) + n) * D + ch] = z16;
      sh.meta_z[ch] = h2f(z16);
      sh.meta_s[ch] = h2f(s16);
    }
  } else {
    const int G = c.cfg.v_group, ng = D / G;
    const int units = BK * ng;
    const int per = units >= kThreads ? 1 : kThreads / units;  // threads per unit
    const int span = G / per;
    for (int base = 0; base < units * per; base += kThreads) {
      const int idx = base + tid;
      const int unit = idx / per, part = idx % per;
      const int j = unit / ng, g = unit % ng;
      float lo = __builtin_inff(), hi = -__builtin_inff();
      int cnt = 0;
      for (int ch = g * G + part * span; ch < g * G + (part + 1) * span; ++ch) {
        if (is_out(j, ch)) continue;
        const float d = dense(j, ch);
        lo = fminf(lo, d);
        hi = fmaxf(hi, d);
        ++cnt;
      }
      for (int m = 1; m < per; m <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, m, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, m, kWave));
        cnt += __shfl_xor(cnt, m, kWave);
      }
      if (part == 0) {
        uint16_t z16, s16;
        meta_from(lo, hi, cnt, L, &z16, &s16);
        c.v_scale[(bh * T + t0 + j) * ng + g] = s16;
        c.v_zero[(bh * T + t0 + j) * ng + g] = z16;
        sh.meta_z[j * ng + g] = h2f(z16);
        sh.meta_s[j * ng + g] = h2f(s16);
      }
    }
  }
  __syncthreads();

  // 5. codes and packing
  if (is_key) {
    const int rowbytes = D * bits / 8;
    uint8_t* out = static_cast<uint8_t*>(c.k_codes) + (bh * T + t0) * rowbytes;
    auto code_of = [&](int j, int ch) -> uint32_t {
      if (is_out(j, ch)) return 0u;
      const float d = dense(j, ch);
      if (c.cfg.k_mode == 1) {
        uint32_t cc = 0;
        for (int k = 0; k < L; ++k) cc += d > sh.mids[ch * 15 + k];
        return cc;
      }
      return (uint32_t)code_uniform(d, sh.meta_z[ch], sh.meta_s[ch], L);
    };
    if (bits == 4) pack_key_rows<D, BK, 4>(out, code_of);
    else if (bits == 3) pack_key_rows<D, BK, 3>(out, code_of);
    else pack_key_rows<D, BK, 2>(out, code_of);
  } else {
    const int vb = bits, tpw = 32 / vb;
    const int G = c.cfg.v_group, ng = D / G;
    uint32_t* out = static_cast<uint32_t*>(c.v_codes) + (bh * (T / tpw) + t0 / tpw) * D;
    const int words = (BK / tpw) * D;
    for (int idx = tid; idx < words; idx += kThreads) {
      const int g = idx / D, ch = idx % D;
      uint32_t w = 0;
      for (int u = 0; u < tpw; ++u) {
        const int j = g * tpw + u;
        int code = 0;
        if (!is_out(j, ch))
          code = code_uniform(dense(j, ch), sh.meta_z[j * ng + ch / G], sh.meta_s[j * ng + ch / G], L);
        w |= (uint32_t)code << (u * vb);
      }
      out[idx] = w;
    }
  }
}

// ---------------------------------------------------------------- tail copy
__global__ void tail_copy_kernel(kvq_cache c, const uint16_t* __restrict__ k_new,
                                 const uint16_t* __restrict__ v_new, int64_t n_new, int64_t src0,
                                 int64_t dst0) {
  const int D = c.cfg.head_dim, Bk = c.cfg.k_block;
  const int64_t rows = n_new - src0;
  const int64_t chunks_per_row = D / 8;
  const int64_t bh = blockIdx.y;
  const int64_t total = rows * chunks_per_row * 2;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int tensor = (int)(i / (rows * chunks_per_row));
    const int64_t r = (i / chunks_per_row) % rows, part = i % chunks_per_row;
    const uint16_t* src = (tensor ? v_new : k_new) + (bh * n_new + src0 + r) * D + part * 8;
    uint16_t* dst = (tensor ? c.v_tail : c.k_tail) + (bh * Bk + dst0 + r) * D + part * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

template <int D, int BK>
hipError_t launch_q(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                    int64_t old_len, int64_t n_new, int64_t n_first, int64_t nblocks, hipStream_t s) {
  if (nblocks * 2 > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)(nblocks * 2), (unsigned)c.cfg.kv_heads, (unsigned)c.cfg.batch);
  hipLaunchKernelGGL((quantize_blocks_kernel<D, BK>), grid, dim3(kThreads), 0, s, c, k_new, v_new,
                     old_len, n_new, n_first);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_init(const kvq_cache& c, hipStream_t s) {
  const int nblk = c.cfg.capacity / c.cfg.k_block;
  const int64_t total = (int64_t)(c.cfg.k_block + nblk) * (c.cfg.head_dim / 2);
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  hipLaunchKernelGGL(rope_init_kernel, dim3(blocks), dim3(256), 0, s, c.rope, c.cfg.head_dim,
                     c.cfg.k_block, nblk, c.cfg.rope_theta);
  return hipGetLastError();
}

hipError_t launch_quantize(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                           int64_t old_len, int64_t n_new, int64_t n_first, int64_t nblocks,
                           hipStream_t s) {
  const int D = c.cfg.head_dim, Bk = c.cfg.k_block;
  if (D == 128 && Bk == 128) return launch_q<128, 128>(c, k_new, v_new, old_len, n_new, n_first, nblocks, s);
  if (D == 128 && Bk == 64) return launch_q<128, 64>(c, k_new, v_new, old_len, n_new, n_first, nblocks, s);
  if (D == 64 && Bk == 128) return launch_q<64, 128>(c, k_new, v_new, old_len, n_new, n_first, nblocks, s);
  if (D == 64 && Bk == 64) return launch_q<64, 64>(c, k_new, v_new, old_len, n_new, n_first, nblocks, s);
  return hipErrorInvalidValue;
}

hipError_t launch_tail_copy(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                            int64_t n_new, int64_t src0, int64_t dst0, hipStream_t s) {
  const int64_t BH = (int64_t)c.cfg.batch * c.cfg.kv_heads;
  if (BH > 65535) return hipErrorInvalidValue;
  const int64_t work = (n_new - src0) * (c.cfg.head_dim / 8) * 2;
  const int blocks = (int)((work + 255) / 256 < 64 ? (work + 255) / 256 : 64);
  hipLaunchKernelGGL(tail_copy_kernel, dim3(blocks > 0 ? blocks : 1, (unsigned)BH), dim3(256), 0, s,
                     c, k_new, v_new, n_new, src0, dst0);
  return hipGetLastError();
}

}  // namespace kvq
