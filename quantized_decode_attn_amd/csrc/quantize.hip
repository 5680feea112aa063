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
  alignas(16) uint8_t krow[BK * D / 2];  // packed key rows of the block (k_bits <= 4)
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


// Uniform code from a dense value with a reciprocal multiply: exact unless the
// quotient lies within 2^-12 of a rounding boundary, which `tie` reports so that the
// caller redoes the element with the correctly rounded divide (code_uniform).  The
// reciprocal and the multiply together are within 2 ulp of the IEEE quotient, far
// inside that margin for |q| <= L + 1; values beyond are clamped first.
__device__ __forceinline__ uint32_t code_fast(float d, float z, float r, float Lf, bool& tie) {
  const float x = d - z;
  const float qv = x * r;
  const float qc = __builtin_amdgcn_fmed3f(qv, -0.75f, Lf + 0.75f);
  const float rr = __builtin_rintf(qc);
  tie |= fabsf(qc - rr) > 0.49975586f;  // 0.5 - 2^-12
  return (uint32_t)__builtin_amdgcn_fmed3f(rr, 0.0f, Lf);
}

__device__ __forceinline__ float recip_or_zero(float s) { return s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s); }

template <int D, int BK, int VB>
__device__ __forceinline__ void value_cells_t(QShared<D, BK>& sh, const kvq_cache& c, int64_t bh, int64_t n,
                                              int L, bool clip, float thr, bool outl) {
  constexpr int P = QShared<D, BK>::kPitch;
  constexpr int TPW = 32 / VB;          // tokens per word (8 or 16)
  constexpr int CW = VB == 4 ? 8 : 4;   // channels per cell
  constexpr int NCC = D / CW;
  constexpr int NTG = BK / TPW;
  const int tid = threadIdx.x;
  const int64_t T = c.cfg.capacity;
  const int G = c.cfg.v_group, ng = D / G;
  const int lpg = G / CW;               // lanes per value group
  const float Lf = (float)L;
  const bool active = tid < NCC * NTG;
  const int tg = tid / NCC, cc = tid % NCC;
  const int ch0 = cc * CW, grp = ch0 / G;

  float x[TPW][CW];
  uint32_t om[TPW];
  float lo[TPW], hi[TPW];
  int cnt[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    lo[u] = __builtin_inff(); hi[u] = -__builtin_inff(); cnt[u] = 0; om[u] = 0;
    if (active) {
      const int j = TPW * tg + u;
      uint32_t hw[CW / 2];
      if constexpr (CW == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sh.tile[j * P + ch0]);
        hw[0] = v.x; hw[1] = v.y; hw[2] = v.z; hw[3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(&sh.tile[j * P + ch0]);
        hw[0] = v.x; hw[1] = v.y;
      }
      if (outl) {
        const uint32_t* mw = &sh.mask[j * (D / 32)];
        om[u] = (mw[ch0 >> 5] >> (ch0 & 31)) & ((1u << CW) - 1u);
      }
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        float v = h2f((uint16_t)(hw[q >> 1] >> (16 * (q & 1))));
        if (clip) v = __builtin_amdgcn_fmed3f(v, -thr, thr);
        x[u][q] = v;
        const bool keep = !((om[u] >> q) & 1u);
        lo[u] = keep ? fminf(lo[u], v) : lo[u];
        hi[u] = keep ? fmaxf(hi[u], v) : hi[u];
        cnt[u] += keep;
      }
    }
  }
  // row statistics of each token over its value group
#pragma unroll
  for (int u = 0; u < TPW; ++u)
    for (int m = 1; m < lpg; m <<= 1) {
      lo[u] = fminf(lo[u], __shfl_xor(lo[u], m, kWave));
      hi[u] = fmaxf(hi[u], __shfl_xor(hi[u], m, kWave));
      if (outl) cnt[u] += __shfl_xor(cnt[u], m, kWave);
    }
  if (active) {
    const int gi = cc % lpg;
    for (int u0 = 0; u0 < TPW; u0 += lpg) {
      const int uu = u0 + gi;
      float l0 = lo[0], h0 = hi[0];
      int c0 = cnt[0];
#pragma unroll
      for (int u = 1; u < TPW; ++u)
        if (uu == u) { l0 = lo[u]; h0 = hi[u]; c0 = cnt[u]; }
      if (uu < TPW) {
        if (!outl) c0 = G;
        uint16_t z16, s16;
        meta_from(l0, h0, c0, L, &z16, &s16);
        const int j = TPW * tg + uu;
        c.v_scale[(bh * T + n * BK + j) * ng + grp] = s16;
        c.v_zero[(bh * T + n * BK + j) * ng + grp] = z16;
        sh.meta_z[j * ng + grp] = h2f(z16);
        sh.meta_s[j * ng + grp] = h2f(s16);
      }
    }
  }
  __syncthreads();
  if (active) {
    uint32_t w[CW];
#pragma unroll
    for (int q = 0; q < CW; ++q) w[q] = 0;
    float zu[TPW], su[TPW];
    bool tie = false;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int j = TPW * tg + u;
      zu[u] = sh.meta_z[j * ng + grp];
      su[u] = sh.meta_s[j * ng + grp];
      const float r = recip_or_zero(su[u]);
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        uint32_t cq = code_fast(x[u][q], zu[u], r, Lf, tie);
        if (outl && ((om[u] >> q) & 1u)) cq = 0;
        w[q] |= cq << (u * VB);
      }
    }
    if (tie) {  // rare: redo with the correctly rounded divide
#pragma unroll
      for (int q = 0; q < CW; ++q) w[q] = 0;
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int q = 0; q < CW; ++q) {
          uint32_t cq = (uint32_t)code_uniform(x[u][q], zu[u], su[u], L);
          if (outl && ((om[u] >> q) & 1u)) cq = 0;
          w[q] |= cq << (u * VB);
        }
    }
    uint32_t* out = static_cast<uint32_t*>(c.v_codes) + (bh * (T / TPW) + n * (BK / TPW) + tg) * D + ch0;
    if constexpr (CW == 8) {
      reinterpret_cast<uint4*>(out)[0] = make_uint4(w[0], w[1], w[2], w[3]);
      reinterpret_cast<uint4*>(out)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      reinterpret_cast<uint4*>(out)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Keys: a cell is 8 tokens x 8 channels, the channels being 4 rotary pairs
// (4a..4a+3 and D/2+4a..D/2+4a+3), so that one cell yields whole packed bytes.
// Cells of one channel set sit in consecutive lanes for the column reductions.
template <int D, int BK>
__device__ __forceinline__ void key_cells(QShared<D, BK>& sh, const kvq_cache& c, int64_t bh, int64_t n, int h,
                                          int L, int kb, bool clip, float thr, bool outl) {
  constexpr int P = QShared<D, BK>::kPitch;
  constexpr int NTG = BK / 8;
  constexpr int NA = D / 8;
  const int tid = threadIdx.x;
  const int64_t T = c.cfg.capacity;
  const bool lut = c.cfg.k_mode == 1;
  const float Lf = (float)L;
  const bool active = tid < NA * NTG;
  const int a = tid / NTG, tg = tid % NTG;
  auto slot_ch = [&](int q) { return q < 4 ? 4 * a + q : D / 2 + 4 * a + q - 4; };

  float x[8][8];
  uint32_t om[8];
  float lo[8], hi[8];
  int cnt[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) { lo[q] = __builtin_inff(); hi[q] = -__builtin_inff(); cnt[q] = 0; }
  if (active) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = 8 * tg + u;
      const uint2 wl = *reinterpret_cast<const uint2*>(&sh.tile[j * P + 4 * a]);
      const uint2 wh = *reinterpret_cast<const uint2*>(&sh.tile[j * P + D / 2 + 4 * a]);
      const uint32_t hw[4] = {wl.x, wl.y, wh.x, wh.y};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float v = h2f((uint16_t)(hw[q >> 1] >> (16 * (q & 1))));
        if (clip) v = __builtin_amdgcn_fmed3f(v, -thr, thr);
        x[u][q] = v;
      }
      om[u] = 0;
      if (outl) {
        const uint32_t* mw = &sh.mask[j * (D / 32)];
        const uint32_t ml = (mw[(4 * a) >> 5] >> ((4 * a) & 31)) & 15u;
        const uint32_t mh = (mw[(D / 2 + 4 * a) >> 5] >> ((D / 2 + 4 * a) & 31)) & 15u;
        om[u] = ml | (mh << 4);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool keep = !((om[u] >> q) & 1u);
        lo[q] = keep ? fminf(lo[q], x[u][q]) : lo[q];
        hi[q] = keep ? fmaxf(hi[q], x[u][q]) : hi[q];
        cnt[q] += keep;
      }
    }
  }
  // column statistics over the whole block: reduce across the NTG lanes of a set
  if (!lut) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int m = 1; m < NTG; m <<= 1) {
        lo[q] = fminf(lo[q], __shfl_xor(lo[q], m, kWave));
        hi[q] = fmaxf(hi[q], __shfl_xor(hi[q], m, kWave));
        if (outl) cnt[q] += __shfl_xor(cnt[q], m, kWave);
      }
    if (active && tg < 8) {
      float l0 = lo[0], h0 = hi[0];
      int c0 = cnt[0];
#pragma unroll
      for (int q = 1; q < 8; ++q)
        if (tg == q) { l0 = lo[q]; h0 = hi[q]; c0 = cnt[q]; }
      if (!outl) c0 = BK;
      uint16_t z16, s16;
      meta_from(l0, h0, c0, L, &z16, &s16);
      const int ch = slot_ch(tg);
      c.k_scale[(bh * (T / BK) + n) * D + ch] = s16;
      c.k_zero[(bh * (T / BK) + n) * D + ch] = z16;
      sh.meta_z[ch] = h2f(z16);
      sh.meta_s[ch] = h2f(s16);
    }
  } else {
    for (int ch = tid; ch < D; ch += kThreads) {
      const uint16_t* lt = c.k_lut + ((int64_t)h * D + ch) * (L + 1);
      for (int k = 0; k < L; ++k) sh.mids[ch * 15 + k] = (h2f(lt[k]) + h2f(lt[k + 1])) * 0.5f;
    }
  }
  __syncthreads();
  if (active) {
    uint32_t w[8];
    if (!lut) {
      float zq[8], sq[8], rq[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        zq[q] = sh.meta_z[slot_ch(q)];
        sq[q] = sh.meta_s[slot_ch(q)];
        rq[q] = recip_or_zero(sq[q]);
      }
      bool tie = false;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        uint32_t wu = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          uint32_t cq = code_fast(x[u][q], zq[q], rq[q], Lf, tie);
          if (outl && ((om[u] >> q) & 1u)) cq = 0;
          const int e = 2 * (q & 3) + (q >> 2);  // element index inside the cell's row bytes
          wu |= cq << (e * kb);
        }
        w[u] = wu;
      }
      if (tie) {  // rare: redo this lane's cell with the correctly rounded divide
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          uint32_t wu = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            uint32_t cq = (uint32_t)code_uniform(x[u][q], zq[q], sq[q], L);
            if (outl && ((om[u] >> q) & 1u)) cq = 0;
            wu |= cq << ((2 * (q & 3) + (q >> 2)) * kb);
          }
          w[u] = wu;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float* md = &sh.mids[slot_ch(q) * 15];
        const int e = 2 * (q & 3) + (q >> 2);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          uint32_t cq = 0;
          for (int k = 0; k < L; ++k) cq += x[u][q] > md[k];
          if (outl && ((om[u] >> q) & 1u)) cq = 0;
          w[u] |= cq << (e * kb);
        }
      }
    }
    // stage the packed bytes of the cell: 8 elements x kb bits = kb bytes per token row
    const int rk = D * kb / 8;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uint8_t* dst = &sh.krow[(8 * tg + u) * rk + a * kb];
      if (kb == 4) {
        *reinterpret_cast<uint32_t*>(dst) = w[u];
      } else if (kb == 2) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w[u];
      } else {
        dst[0] = (uint8_t)w[u];
        dst[1] = (uint8_t)(w[u] >> 8);
        dst[2] = (uint8_t)(w[u] >> 16);
      }
    }
  }
  __syncthreads();
  // coalesced 16-byte stores of the block's rows
  {
    const int rk = D * kb / 8;
    uint8_t* out = static_cast<uint8_t*>(c.k_codes) + (bh * T + n * BK) * rk;
    for (int idx = tid; idx < BK * rk / 16; idx += kThreads)
      reinterpret_cast<uint4*>(out)[idx] = reinterpret_cast<const uint4*>(sh.krow)[idx];
  }
}

// Values: a cell is (32/v_bits) consecutive tokens x CW channels, so that each of
// its CW channels yields one packed word; the cells of one value group sit in
// consecutive lanes for the row reductions.
template <int D, int BK>
__device__ __forceinline__ void value_cells(QShared<D, BK>& sh, const kvq_cache& c, int64_t bh, int64_t n,
                                            int L, int vb, bool clip, float thr, bool outl) {
  if (vb == 4)
    value_cells_t<D, BK, 4>(sh, c, bh, n, L, clip, thr, outl);
  else
    value_cells_t<D, BK, 2>(sh, c, bh, n, L, clip, thr, outl);
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

  // 4-5. statistics, metadata, codes and packing, one register cell per thread
  if (is_key)
    key_cells<D, BK>(sh, c, bh, n, h, L, bits, clip, thr, ko > 0);
  else
    value_cells<D, BK>(sh, c, bh, n, L, bits, clip, thr, ko > 0);
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
