// quantize_block.h -- the block quantizer shared by the key and value kernels.
//
// Pages cited (title, address):
//   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
//   [UQ]   "大模型长上下文推理优化：4-bit KV Cache量化技术解析与部署实践", mlqm.cn/news/1064729
//   [TQ]   "TurboQuant：突破大模型推理瓶颈的KVCache量化技术解析", mlqm.cn/news/1002276
//
// One workgroup (256 threads, 4 waves) owns one (b, kv-head, block) of one tensor.
// The k_block x head_dim fp16 tile is staged once in LDS; the steps, in the order the
// pages give them:
//   1. dense-and-sparse split: per token vector, the ko largest |x| (ties to the lower
//      column) go to the CSR ([KVC3] "Per-Vector Dense-and-Sparse Quantization");
//      their tile entries are then overwritten with a quiet NaN, which fminf/fmaxf
//      skip, so the statistics below exclude them at no cost;
//   2. clip threshold: exact q-quantile of |x| over the tile (outliers included) by
//      radix selection on the 15-bit fp16 magnitudes, linear interpolation in fp64
//      ([UQ] section 4.2); for high quantiles the selection runs over a short list of
//      candidates that provably holds both order statistics;
//   3. statistics: keys per channel over the block ([KVC3] "Per-Channel Key
//      Quantization", before RoPE per "Pre-RoPE Key Quantization"), values per token
//      over channel groups ([KVC3] "Quanto 的量化原理"); fp16 zero rounded down and
//      fp16 scale rounded up.  Clipping is monotone, so the statistics of the clipped
//      values are the clipped statistics;
//   4. codes: round-half-even((d - zero) / scale) clamped to [0, 2^bits - 1]
//      (round(x/scale) of [TQ] section 4.2), or the nearest codebook entry
//      ([KVC3] "Non-Uniform KV Cache Quantization"); outlier positions get code 0.
//
// Steps 1 and 2 work on the values each thread staged, still in registers; each
// thread holds one register cell of the tile (8 x 8 elements for keys, 8 x 8 or
// 16 x 4 for values) from step 3 on.  Both kernels are compiled for four waves per
// SIMD (at most 128 registers), which the tile's LDS footprint also allows.  The code is computed as rint((d - z) * rcp(s)),
// which differs from the correctly rounded quotient by a few ulp only; a quotient
// within 2^-17 of a rounding boundary is decided exactly from the residual of the
// nearest half-integer (code_near), so the stored bits are those of the exact
// definition, rint of the IEEE fp32 quotient.  Clipping to
// [-thr, thr] is applied as a clamp of the quotient to [q(-thr), q(thr)]: the
// quotient is monotone in d, so this equals the quotient of the clipped value.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace qb {

constexpr int kThreads = 256;
constexpr uint16_t kMarkNaN = 0x7E00;  // fp16 quiet NaN marking an outlier in the tile
// A quotient closer than 2^-17 to a rounding boundary is decided exactly.  The fast
// quotient (d - z) * rcp(s) is within |q| 2^-22 of the correctly rounded one (rcp is
// good to 1 ulp, the product and the IEEE quotient to half an ulp each), i.e. within
// 2^-18 for the clamped |q| <= 16, so every other element rounds the same either way.
constexpr float kTieMargin = 0.49999237f;  // 0.5 - 2^-17

// ---------------------------------------------------------------- block reductions
struct Red {
  uint32_t u[kThreads / kWave];
  int sh_bin;
  uint32_t sh_below;
  float thr;
};

__device__ inline uint32_t block_sum_u32(uint32_t v, Red& r) {
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
__device__ inline uint32_t block_min_u32(uint32_t v, Red& r) {
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
__device__ inline void find_bin(const uint32_t* hist, int nbins, uint32_t rank, int* out_bin,
                                uint32_t* out_below, Red& r) {
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
      r.sh_bin = b;
      r.sh_below = below;
    }
  }
  __syncthreads();
  *out_bin = r.sh_bin;
  *out_below = r.sh_below;
}

// The bin holding the element of rank `rank_top` counted from the largest (0-based),
// scanning from the top bin down; returns the bin and the count of elements in the
// bins above it.  Bins below the answer need not be counted.  Wave 0 scans, the
// result is broadcast through LDS.
__device__ inline void find_bin_top(const uint32_t* hist, int nbins, uint32_t rank_top, int* out_bin,
                                    uint32_t* out_above, Red& r) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = nbins / kWave;
    const int hi = nbins - lane * per;  // lane covers bins [hi - per, hi), top lanes first
    uint32_t local = 0;
    for (int k = 1; k <= per; ++k) local += hist[hi - k];
    uint32_t incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      uint32_t o = (uint32_t)__shfl_up((int)incl, d, kWave);
      if (lane >= d) incl += o;
    }
    const uint64_t over = __ballot(incl > rank_top);
    const int first = __ffsll((unsigned long long)over) - 1;
    if (lane == first) {
      uint32_t above = incl - local;
      int b = hi - 1;
      for (int k = 1; k <= per; ++k) {
        const uint32_t h = hist[hi - k];
        if (above + h > rank_top) { b = hi - k; break; }
        above += h;
      }
      r.sh_bin = b;
      r.sh_below = above;
    }
  }
  __syncthreads();
  *out_bin = r.sh_bin;
  *out_above = r.sh_below;
}

// ---------------------------------------------------------------- cross-lane min/max
// One v_min_f32 / v_max_f32 with a DPP source (the s_nop covers the VALU-write to
// DPP-read hazard).  Written out because the compiler otherwise brackets every
// cross-lane operand with NaN-quieting moves; the operands here are never signaling
// NaNs (converted fp16 values, infinities), and the hardware min/max return the
// other operand for a quiet NaN.
#define KVQ_DPP_MINMAX(NAME, OP, CTRL)                                                          \
  __device__ __forceinline__ float NAME(float v) {                                              \
    float r;                                                                                    \
    asm("s_nop 1\n\t" OP " %0, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v)); \
    return r;                                                                                   \
  }
KVQ_DPP_MINMAX(min_x1, "v_min_f32_dpp", "quad_perm:[1,0,3,2]")
KVQ_DPP_MINMAX(min_x2, "v_min_f32_dpp", "quad_perm:[2,3,0,1]")
KVQ_DPP_MINMAX(min_hm, "v_min_f32_dpp", "row_half_mirror")
KVQ_DPP_MINMAX(min_rm, "v_min_f32_dpp", "row_mirror")
KVQ_DPP_MINMAX(max_x1, "v_max_f32_dpp", "quad_perm:[1,0,3,2]")
KVQ_DPP_MINMAX(max_x2, "v_max_f32_dpp", "quad_perm:[2,3,0,1]")
KVQ_DPP_MINMAX(max_hm, "v_max_f32_dpp", "row_half_mirror")
KVQ_DPP_MINMAX(max_rm, "v_max_f32_dpp", "row_mirror")
#undef KVQ_DPP_MINMAX

// Minimum / maximum over aligned groups of N lanes (N in {1,2,4,8,16}) for every lane.
template <int N>
__device__ __forceinline__ float lanes_min(float v) {
  if constexpr (N >= 2) v = min_x1(v);
  if constexpr (N >= 4) v = min_x2(v);
  if constexpr (N >= 8) v = min_hm(v);
  if constexpr (N >= 16) v = min_rm(v);
  return v;
}
template <int N>
__device__ __forceinline__ float lanes_max(float v) {
  if constexpr (N >= 2) v = max_x1(v);
  if constexpr (N >= 4) v = max_x2(v);
  if constexpr (N >= 8) v = max_hm(v);
  if constexpr (N >= 16) v = max_rm(v);
  return v;
}

// Packed fp16 minimum / maximum of two elements per register.  Minimum and maximum of
// fp16 values are exact in fp16, and in IEEE mode a quiet NaN operand (the outlier mark)
// yields the other operand, as fminf/fmaxf do.  Written out so that the compiler adds no
// NaN-quieting operations around the loaded operands (never signaling NaNs here).
__device__ __forceinline__ uint32_t pk_min_h(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t pk_max_h(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
constexpr uint32_t kPkPosInf = 0x7C007C00u, kPkNegInf = 0xFC00FC00u;

// Element k (0 or 1) of a packed fp16 pair.
__device__ __forceinline__ _Float16 half_of(uint32_t w, int k) {
  return __builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * k)));
}

// ---------------------------------------------------------------- scalar pieces

// fp16 zero = min rounded down, fp16 scale = (max - zero) / L rounded up; a group
// with no dense value (lo > hi) gets zero 0 and scale 0.
__device__ __forceinline__ void meta_from(float lo, float hi, int L, uint16_t* z16, uint16_t* s16) {
  if (!(lo <= hi)) { lo = 0.0f; hi = 0.0f; }
  lo = lo + 0.0f;
  hi = hi + 0.0f;
  *z16 = f2h_rd(lo);
  const float range = hi - h2f(*z16);
  const float s32 = range / (float)L;
  *s16 = f2h_ru(s32);
}

__device__ __forceinline__ float recip_or_zero(float s) {
  return s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
}

// Quotient clamp bounds for one (zero, reciprocal): [0, L] without clipping, else
// [q(-thr), q(thr)] clamped to [0, L].
template <bool CLIP>
__device__ __forceinline__ void quotient_bounds(float z, float r, float Lf, float thr, float* a, float* b) {
  if constexpr (CLIP) {
    *a = __builtin_amdgcn_fmed3f((-thr - z) * r, 0.0f, Lf);
    *b = __builtin_amdgcn_fmed3f((thr - z) * r, 0.0f, Lf);
  } else {
    *a = 0.0f;
    *b = Lf;
  }
}

// Fast code of one element as an integral float; `tie` collects quotients too close
// to a rounding boundary.  The quotient is clamped to [a, b] = [0, L], or with
// clipping to the quotients of -thr and thr.
template <bool OUTL, bool CLIP>
__device__ __forceinline__ float code_fast(float d, float z, float r, float a, float b, bool& near, float& qc) {
  const float x = d - z;
  qc = x * r;
  qc = __builtin_amdgcn_fmed3f(qc, a, b);
  if constexpr (OUTL) qc = (d != d) ? 0.0f : qc;
  const float rr = __builtin_rintf(qc);
  near = fabsf(qc - rr) > kTieMargin;
  return rr;
}

// The same from the element's fp16 bits: d - z is one mixed-precision FMA (d * 1 - z,
// rounded once: the IEEE fp32 subtraction of the converted value), and an outlier mark
// (NaN) propagates to the difference.
template <bool OUTL, bool CLIP>
__device__ __forceinline__ float code_fast_h(_Float16 h, float z, float r, float a, float b, bool& near, float& qc) {
  const float x = __builtin_fmaf((float)h, 1.0f, -z);
  qc = x * r;
  qc = __builtin_amdgcn_fmed3f(qc, a, b);
  if constexpr (OUTL) qc = (x != x) ? 0.0f : qc;
  const float rr = __builtin_rintf(qc);
  near = fabsf(qc - rr) > kTieMargin;
  return rr;
}

// Byte k of w replaced by the integral value c (0..255).
__device__ __forceinline__ uint32_t put_byte(float c, uint32_t k, uint32_t w) {
  return __builtin_amdgcn_cvt_pk_u8_f32(c, k, w);
}

// Exact code of one element (the fallback).
// Exact code of an element whose fast quotient qc lies within 2^-17 of the half-integer
// h = floor(qc) + 1/2, without a divide: the code is rint of the IEEE quotient
// q = fl(num / s), num = fp32(d - z).  The residual r = num - h s is exact (h s has at
// most 17 significant bits and cancels with num), and q == h exactly when
// |r| <= s ulp(h) / 2 (h has few mantissa bits, so ties of the quotient's rounding go to
// h); otherwise q lies on r's side of h.  A quotient equal to h rounds half to even.
// (h = 1/2, the one power of two, rounds down on a tie and on the side below, so the
// narrower lower half-ulp there does not matter.)
template <bool OUTL, bool CLIP>
__device__ __forceinline__ float code_near(float d, float z, float s, float qc, float Lf, float thr) {
  if constexpr (OUTL)
    if (d != d) return 0.0f;
  if constexpr (CLIP) d = fminf(fmaxf(d, -thr), thr);
  if (s == 0.0f) return 0.0f;
  const float num = d - z;
  const float k = __builtin_floorf(qc);
  const float h = k + 0.5f;
  const float r = __builtin_fmaf(-h, s, num);
  const float hu = __builtin_amdgcn_ldexpf(s, __builtin_amdgcn_frexp_expf(h) - 25);  // s ulp(h) / 2
  const float even = k + (float)((int)k & 1);
  const float code = r > hu ? k + 1.0f : (r < -hu ? k : even);
  return fminf(fmaxf(code, 0.0f), Lf);
}

// ---------------------------------------------------------------- phases 1-2b
// Thread tid stages chunks i < NC of 8 consecutive values: chunk i is token row
// i * (kThreads / LPR) + tid / LPR, columns 8 (tid % LPR) .. +7, so the LPR = D / 8
// threads of a row are consecutive lanes.  The outlier search and the clip's
// candidate collection run on these registers; the tile in LDS is written once.
template <int D, int BK>
struct Stage {
  static constexpr int LPR = D / 8;                     // threads per token row
  static constexpr int RPS = kThreads / LPR;            // rows per chunk index
  static constexpr int NC = BK / RPS;                   // chunks per thread
  static_assert(NC * RPS == BK && NC * kThreads * 8 == BK * D, "tile split");
};

// Largest and middle of three (v_max3_u32 / v_med3_u32 after instruction selection).
__device__ __forceinline__ uint32_t umax3(uint32_t a, uint32_t b, uint32_t c) { return max(max(a, b), c); }
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

// Unsigned maximum over aligned groups of N lanes (N = 8 or 16).
template <int N>
__device__ __forceinline__ uint32_t lanes_max_u32(uint32_t v) {
  static_assert(N == 8 || N == 16, "rows of 8 or 16 lanes");
  v = max(v, dpp_u<kDppQuadXor1>(v));
  v = max(v, dpp_u<kDppQuadXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  if constexpr (N == 16) v = max(v, dpp_u<kDppRowMirror>(v));
  return v;
}

// Loads the thread's chunks (rows from the old tail below old_len, else from the new
// input) and writes them to the tile.
template <int D, int BK>
__device__ __forceinline__ void stage_chunks(uint4 (&v)[BK * D / 8 / kThreads], uint16_t* tile, const uint16_t* tail,
                                             const uint16_t* src_new, int64_t bh, int64_t t0, int64_t old_len,
                                             int64_t n_new) {
  using S = Stage<D, BK>;
  constexpr int P = D + 8;
  const int64_t tail0 = (old_len / BK) * BK;
  const int r0 = threadIdx.x / S::LPR, part = threadIdx.x % S::LPR;
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  if (t0 >= old_len) {
    // the whole block comes from the new tokens (every block but the first after an
    // append that left a tail): one block base and 32-bit lane offsets
    const uint16_t* blk = src_new + (bh * n_new + (t0 - old_len)) * D;
#pragma unroll
    for (int i = 0; i < S::NC; ++i) {
      const uint32_t off = (uint32_t)((i * S::RPS + r0) * D + part * 8) * 2u;
      // the new fp16 tokens are read once: non-temporal loads
      const u4v x = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(reinterpret_cast<const char*>(blk) + off));
      v[i] = make_uint4(x.x, x.y, x.z, x.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < S::NC; ++i) {
      const int j = i * S::RPS + r0;
      const int64_t t = t0 + j;
      const uint16_t* row = t < old_len ? tail + (bh * BK + (t - tail0)) * D
                                        : src_new + (bh * n_new + (t - old_len)) * D;
      const u4v x = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(row + part * 8));
      v[i] = make_uint4(x.x, x.y, x.z, x.w);
    }
  }
#pragma unroll
  for (int i = 0; i < S::NC; ++i)
    *reinterpret_cast<uint4*>(&tile[(i * S::RPS + r0) * P + part * 8]) = v[i];
}

// Step 1 from registers: per token row the ko largest keys |x| bits << 8 | 255 - column
// (unique within a row, so ties go to the lower column), one row maximum per round,
// the rounds of all the thread's rows interleaved.  The lane owning an outlier's
// column stages it in ocol/oval (ascending column order within the row, value read
// back from the tile it wrote itself); the columns are returned packed a byte each
// for the marking after the clip.
template <int D, int BK, int KO>
__device__ __forceinline__ void row_outliers(const uint4 (&v)[BK * D / 8 / kThreads], const uint16_t* tile, int ko_rt,
                                             uint8_t* ocol, uint16_t* oval, uint32_t (&colpk)[BK * D / 8 / kThreads]) {
  using S = Stage<D, BK>;
  constexpr int P = D + 8;
  constexpr int KMAX = KO > 0 ? KO : 4;  // outlier slots a row can hold
  const int ko = KO > 0 ? KO : ko_rt;
  constexpr int G = S::NC < 2 ? S::NC : 2;  // rows searched together (register budget)
  const int r0 = threadIdx.x / S::LPR, part = threadIdx.x % S::LPR;
#pragma unroll
  for (int i0 = 0; i0 < S::NC; i0 += G) {
    uint32_t key[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 vi = v[i0 + g];
      const uint32_t w[4] = {vi.x, vi.y, vi.z, vi.w};
#pragma unroll
      for (int k = 0; k < 8; ++k)
        key[g][k] = (((w[k >> 1] >> (16 * (k & 1))) & 0x7fffu) << 8) | (uint32_t)(255 - (8 * part + k));
    }
    uint32_t sel[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) sel[g][0] = sel[g][1] = sel[g][2] = sel[g][3] = 0u;
    if (KO == 1 || KO == 2 || (KO < 0 && ko <= 2)) {
      // the lane's two largest keys by a merge tree, then the row's largest, then the
      // row's largest among the other lanes' first and the owner's second
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // groups {0,1,2}, {3,4,5}, {6,7}: top of each by max3 / max, second by med3 / min;
        // the lane's second is the larger of the middle top and the largest second (a
        // group's second is below its own top, and every top but the largest is at most
        // the middle one)
        const uint32_t* k8 = key[g];
        const uint32_t t0 = umax3(k8[0], k8[1], k8[2]);
        const uint32_t s0 = umed3(k8[0], k8[1], k8[2]);
        const uint32_t t1 = umax3(k8[3], k8[4], k8[5]);
        const uint32_t s1 = umed3(k8[3], k8[4], k8[5]);
        const uint32_t t2 = max(k8[6], k8[7]), s2 = min(k8[6], k8[7]);
        const uint32_t m1 = umax3(t0, t1, t2);
        const uint32_t m2 = max(umed3(t0, t1, t2), umax3(s0, s1, s2));
        const uint32_t M1 = lanes_max_u32<S::LPR>(m1);
        sel[g][0] = M1;
        if (ko == 2) sel[g][1] = lanes_max_u32<S::LPR>(m1 == M1 ? m2 : m1);
      }
    } else {
      uint32_t prev[G];
#pragma unroll
      for (int g = 0; g < G; ++g) prev[g] = 0xffffffffu;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < ko) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            uint32_t m = 0u;
#pragma unroll
            for (int k = 0; k < 8; ++k) m = max(m, key[g][k] < prev[g] ? key[g][k] : 0u);
            m = lanes_max_u32<S::LPR>(m);
            sel[g][r] = m;
            prev[g] = m;
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = i0 + g;
      const int j = i * S::RPS + r0;
      int cols[4];
      colpk[i] = 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cols[r] = 255 - (int)(sel[g][r] & 0xffu);
        if (r < KMAX) colpk[i] |= (uint32_t)(cols[r] & 0xff) << (8 * r);
      }
#pragma unroll
      for (int r = 0; r < KMAX; ++r) {
        if (r < ko && (cols[r] >> 3) == part) {
          int rank = 0;
#pragma unroll
          for (int q = 0; q < KMAX; ++q) rank += (q < ko && cols[q] < cols[r]) ? 1 : 0;
          ocol[j * 4 + rank] = (uint8_t)cols[r];
          oval[j * 4 + rank] = tile[j * P + cols[r]];
        }
      }
    }
  }
}

// Writes the block's CSR slice staged in ocol/oval (consecutive threads) and its
// row pointers (ko entries per token).  col_out / val_out point at the slot's Bk * ko
// entries, rowptr at the row-pointer array the tokens t_base + j index (the (b, h)
// row's T + 1 entries with t_base = the block's first token in the dense layout; the
// slot's own Bk + 1 with t_base = 0 in the paged one).
template <int BK, int KO>
__device__ __forceinline__ void write_csr(const uint8_t* ocol, const uint16_t* oval, int32_t* rowptr, uint8_t* col_out,
                                          uint16_t* val_out, int64_t t_base, int ko_rt) {
  const int ko = KO > 0 ? KO : ko_rt;
  for (int idx = threadIdx.x; idx < BK * ko; idx += kThreads) {
    const int j = idx / ko, r = idx % ko;
    col_out[idx] = ocol[j * 4 + r];
    val_out[idx] = oval[j * 4 + r];
  }
  for (int j = threadIdx.x; j < BK; j += kThreads) {
    const int64_t t = t_base + j;
    rowptr[t + 1] = (int32_t)((t + 1) * ko);
    if (t == 0) rowptr[0] = 0;
  }
}

// The outlier positions get the quiet NaN in the tile (each by the thread that staged
// the position).
template <int D, int BK, int KO>
__device__ __forceinline__ void mark_outliers(uint16_t* tile, const uint32_t (&colpk)[BK * D / 8 / kThreads], int ko_rt) {
  using S = Stage<D, BK>;
  constexpr int P = D + 8;
  constexpr int KMAX = KO > 0 ? KO : 4;
  const int ko = KO > 0 ? KO : ko_rt;
  const int r0 = threadIdx.x / S::LPR, part = threadIdx.x % S::LPR;
#pragma unroll
  for (int i = 0; i < S::NC; ++i)
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      const int col = (int)((colpk[i] >> (8 * r)) & 0xffu);
      if (r < ko && (col >> 3) == part) tile[(i * S::RPS + r0) * P + col] = kMarkNaN;
    }
}

// ---------------------------------------------------------------- phase 2b: clip
// Exact order statistics of |x| (15-bit magnitudes) over the whole tile, outliers
// included: the element of rank kr = floor(q (n - 1)) and the next one, then
// t = v_kr + frac * (v_kr+1 - v_kr) in fp64, each operation rounded separately.
constexpr int kCandCap = 256;  // clip candidates per wave
struct ClipSmem {
  uint32_t hist[256];
  uint32_t ncand[kThreads / kWave];
  alignas(16) uint16_t cand[kThreads / kWave][kCandCap];  // (kept-key norms when not clipping)
};

// The largest 15-bit magnitude of each of the thread's staged chunks.
template <int NC>
__device__ __forceinline__ void chunk_maxima(const uint4 (&v)[NC], uint32_t (&cmax)[NC]) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const us2 a = __builtin_elementwise_max(__builtin_bit_cast(us2, v[i].x & 0x7fff7fffu),
                                            __builtin_bit_cast(us2, v[i].y & 0x7fff7fffu));
    const us2 b = __builtin_elementwise_max(__builtin_bit_cast(us2, v[i].z & 0x7fff7fffu),
                                            __builtin_bit_cast(us2, v[i].w & 0x7fff7fffu));
    const us2 m = __builtin_elementwise_max(a, b);
    cmax[i] = m.x > m.y ? m.x : m.y;
  }
}

// Candidates (cmax: the thread's chunk maxima): when the target's rank from the top,
// rank_top, is below kThreads, each wave takes kk = ceil((rank_top + 1) / 4) and the
// kk-th largest of its lanes' maxima m_w (a bitwise search on ballot counts); at least
// kk of the wave's values are >= m_w, so at least rank_top + 1 values of the tile are
// >= T = min_w m_w, and the target and the next larger value are among the values
// >= T.  Each wave appends its values >= T to its own list, visiting only the chunks
// whose maximum reaches T (read back from the tile the thread staged).  Returns false
// (for every thread) when the bound does not apply or a list overflowed.
template <int D, int BK>
__device__ __forceinline__ bool clip_candidates(const uint16_t* tile, const uint32_t (&cmax)[BK * D / 8 / kThreads],
                                                uint32_t rank_top, ClipSmem& cs, Red& red) {
  using S = Stage<D, BK>;
  constexpr int P = D + 8;
  if (rank_top >= (uint32_t)kThreads) return false;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t gmax = 0u;
#pragma unroll
  for (int i = 0; i < S::NC; ++i) gmax = max(gmax, cmax[i]);
  const uint32_t kk = (rank_top + 4) / 4;
  uint32_t pre = 0u;
#pragma unroll
  for (int bit = 14; bit >= 0; --bit) {
    const uint32_t cand = pre | (1u << bit);
    if ((uint32_t)__popcll(__ballot(gmax >= cand)) >= kk) pre = cand;
  }
  if (lane == 0) {
    red.u[wave] = pre;
    cs.ncand[wave] = 0u;
  }
  __syncthreads();
  uint32_t T = red.u[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) T = min(T, red.u[w]);
  uint32_t mask = 0u;
#pragma unroll
  for (int i = 0; i < S::NC; ++i) mask |= (cmax[i] >= T ? 1u : 0u) << i;
  uint16_t* lst = cs.cand[wave];
  const int r0 = threadIdx.x / S::LPR, part = threadIdx.x % S::LPR;
  while (mask != 0u) {
    const int i = __builtin_ctz(mask);
    mask &= mask - 1u;
    const uint4 c4 = *reinterpret_cast<const uint4*>(&tile[(i * S::RPS + r0) * P + part * 8]);
    const uint32_t w[4] = {c4.x, c4.y, c4.z, c4.w};
    uint32_t x[8], n = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = (w[k >> 1] >> (16 * (k & 1))) & 0x7fffu;
      n += x[k] >= T ? 1u : 0u;
    }
    uint32_t pos = atomicAdd(&cs.ncand[wave], n);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (x[k] >= T) {
        if (pos < (uint32_t)kCandCap) lst[pos] = (uint16_t)x[k];
        ++pos;
      }
    }
  }
  __syncthreads();
  bool ok = true;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) ok = ok && cs.ncand[w] <= (uint32_t)kCandCap;
  return ok;
}

// The fp64 interpolation between the two order statistics, by thread 0, broadcast.
__device__ __forceinline__ float clip_interp(uint32_t vk, uint32_t vk1, bool last, double frac, Red& red) {
  if (threadIdx.x == 0) {
    float t;
    const double v0 = (double)h2f((uint16_t)vk);
    if (last) {
      t = (float)v0;
    } else {
      const double v1 = (double)h2f((uint16_t)vk1);
      const double diff = v1 - v0;
      const double prod = frac * diff;
      const double sum = v0 + prod;
      t = (float)sum;
    }
    red.thr = t;
  }
  __syncthreads();
  return red.thr;
}

__device__ __forceinline__ void quantile_rank(float quantile, int nel, int64_t* kr, double* frac, uint32_t* rank_top) {
  const double pos = (double)quantile * (double)(nel - 1);
  *kr = (int64_t)floor(pos);
  *frac = pos - (double)*kr;
  *rank_top = (uint32_t)(nel - 1 - *kr);
}

// The two order statistics from the candidate lists: radix selection over the lists
// only, from the top (8 high bits, then the 7 low bits inside the bin); the next
// larger value is vk again unless exactly rank_top values exceed vk, then the
// smallest candidate above vk.
template <int NEL>
__device__ __forceinline__ float clip_from_candidates(ClipSmem& cs, Red& red, float quantile) {
  int64_t kr;
  double frac;
  uint32_t rank_top;
  quantile_rank(quantile, NEL, &kr, &frac, &rank_top);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t nw = cs.ncand[wave];
  const uint16_t* lst = cs.cand[wave];
  for (int i = tid; i < 256; i += kThreads) cs.hist[i] = 0u;
  __syncthreads();
  for (uint32_t e = lane; e < nw; e += kWave) atomicAdd(&cs.hist[lst[e] >> 7], 1u);
  __syncthreads();
  int bin1;
  uint32_t above1;
  find_bin_top(cs.hist, 256, rank_top, &bin1, &above1, red);
  for (int i = tid; i < 128; i += kThreads) cs.hist[i] = 0u;
  __syncthreads();
  for (uint32_t e = lane; e < nw; e += kWave) {
    const uint32_t x = lst[e];
    if ((int)(x >> 7) == bin1) atomicAdd(&cs.hist[x & 127u], 1u);
  }
  __syncthreads();
  int bin2;
  uint32_t above2;
  find_bin_top(cs.hist, 128, rank_top - above1, &bin2, &above2, red);
  const uint32_t vk = ((uint32_t)bin1 << 7) | (uint32_t)bin2;
  uint32_t vk1 = vk;
  if (rank_top >= 1u && above1 + above2 == rank_top) {
    uint32_t m = 0xffffffffu;
    for (uint32_t e = lane; e < nw; e += kWave) {
      const uint32_t x = lst[e];
      m = x > vk ? min(m, x) : m;
    }
    vk1 = block_min_u32(m, red);
  }
  return clip_interp(vk, vk1, rank_top == 0u, frac, red);
}

// The same statistics from the whole tile (when the candidate bound does not
// apply): radix selection of rank kr over all elements, 8 high bits then 7 low bits.
// `group_max`: the largest magnitude among the values this thread staged.  Every
// thread's values form a disjoint group, so at least kThreads values are >= the
// smallest group maximum m; when the target's rank counted from the top is below
// kThreads, the target is >= m, and the histogram pass skips every bin below m's.
template <int D, int BK>
__device__ __forceinline__ float clip_from_tile(const uint16_t* tile, ClipSmem& cs, Red& red, float quantile,
                                                uint32_t group_max) {
  constexpr int P = D + 8;
  constexpr int NEL = BK * D;
  constexpr int kChunks = NEL / 8;
  const int tid = threadIdx.x;
  int64_t kr;
  double frac;
  uint32_t rank_top;
  quantile_rank(quantile, NEL, &kr, &frac, &rank_top);
  auto chunk = [&](int idx) -> uint4 {
    const int j = idx / (D / 8), part = idx % (D / 8);
    return *reinterpret_cast<const uint4*>(&tile[j * P + part * 8]);
  };
  for (int i = tid; i < 256; i += kThreads) cs.hist[i] = 0;
  const uint32_t low_bin = rank_top < (uint32_t)kThreads ? block_min_u32(group_max, red) >> 7 : 0u;
  __syncthreads();
  // pass 1: top 8 of the 15 magnitude bits, bins >= low_bin only
  for (int idx = tid; idx < kChunks; idx += kThreads) {
    const uint4 w = chunk(idx);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t key = (ws[k >> 1] >> (16 * (k & 1))) & 0x7fffu;
      if ((key >> 7) >= low_bin) atomicAdd(&cs.hist[key >> 7], 1u);
    }
  }
  __syncthreads();
  int bin1;
  uint32_t above1;
  find_bin_top(cs.hist, 256, rank_top, &bin1, &above1, red);
  const uint32_t below1 = (uint32_t)NEL - above1 - cs.hist[bin1];
  __syncthreads();
  // pass 2: low 7 bits inside the selected bin
  for (int i = tid; i < 256; i += kThreads) cs.hist[i] = 0;
  __syncthreads();
  for (int idx = tid; idx < kChunks; idx += kThreads) {
    const uint4 w = chunk(idx);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t key = (ws[k >> 1] >> (16 * (k & 1))) & 0x7fffu;
      if ((int)(key >> 7) == bin1) atomicAdd(&cs.hist[key & 127], 1u);
    }
  }
  __syncthreads();
  int bin2;
  uint32_t below2;
  find_bin(cs.hist, 128, (uint32_t)kr - below1, &bin2, &below2, red);
  const uint32_t vk = ((uint32_t)bin1 << 7) | (uint32_t)bin2;
  // the next order statistic: vk again if it repeats past rank kr, else the smallest
  // magnitude above vk.  Every sub-bin of bin1 is one magnitude, so that is the next
  // occupied sub-bin; only when bin1 holds nothing above vk does a pass over the tile
  // find it.
  uint32_t vk1 = vk;
  if (kr + 1 < NEL && below1 + below2 + cs.hist[bin2] < (uint32_t)(kr + 2)) {
    const uint32_t cand = (tid < 128 && tid > bin2 && cs.hist[tid] != 0u) ? (uint32_t)tid : 0xffffffffu;
    const uint32_t nb = block_min_u32(cand, red);
    if (nb != 0xffffffffu) {
      vk1 = ((uint32_t)bin1 << 7) | nb;
    } else {
      uint32_t gt_min = 0xffffffffu;
      for (int idx = tid; idx < kChunks; idx += kThreads) {
        const uint4 w = chunk(idx);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t key = (ws[k >> 1] >> (16 * (k & 1))) & 0x7fffu;
          gt_min = key > vk ? min(gt_min, key) : gt_min;
        }
      }
      vk1 = block_min_u32(gt_min, red);
    }
  }
  return clip_interp(vk, vk1, kr + 1 >= NEL, frac, red);
}

// ---------------------------------------------------------------- shared memory
template <int D, int BK>
struct KeyMeta {  // per channel
  float z[D], r[D], s[D], a[D], b[D];
};
template <int D, int BK>
struct ValueMeta {  // per (group, token), groups of at least 16 channels
  float z[(D / 16) * BK], r[(D / 16) * BK], s[(D / 16) * BK], a[(D / 16) * BK], b[(D / 16) * BK];
};

template <int D, int BK>
struct KeySmem {
  static constexpr int kRowPitchMax = D / 2 + 16;  // packed key row (<= 4 bits) + padding
  union alignas(16) {
    uint16_t tile[BK * (D + 8)];
    struct {
      KeyMeta<D, BK> meta;
      alignas(16) uint8_t krow[BK * kRowPitchMax];
      float mids[D * 15];
    } out;
  } u;
  uint8_t ocol[BK * 4];
  uint16_t oval[BK * 4];
  ClipSmem clip;
  Red red;
};

template <int D, int BK>
struct ValueSmem {
  union alignas(16) {
    uint16_t tile[BK * (D + 8)];
    ValueMeta<D, BK> meta;
  } u;
  uint8_t ocol[BK * 4];
  uint16_t oval[BK * 4];
  ClipSmem clip;
  Red red;
};

// Steps 1, 2 and 2b for one tile; returns the clip threshold (0 without clipping).
// The tile is written raw; the outliers are marked after the clip (which counts them).
template <int D, int BK, int KO, bool CLIP>
__device__ __forceinline__ float prepare_tile(uint16_t* tile, uint8_t* ocol, uint16_t* oval, ClipSmem& cs, Red& red,
                                              const kvq_cache& c, bool is_key, const uint16_t* src_new,
                                              int64_t bh, int64_t n, int64_t g, int64_t old_len, int64_t n_new) {
  using S = Stage<D, BK>;
  const int64_t T = c.cfg.capacity;
  const int64_t t0 = n * BK;
  uint4 v[S::NC];
  stage_chunks<D, BK>(v, tile, is_key ? c.k_tail : c.v_tail, src_new, bh, t0, old_len, n_new);
  const int ko = kout_of(c.cfg);
  uint32_t gmax = 0u;
  bool fast = false;
  if constexpr (CLIP) {
    int64_t kr;
    double frac;
    uint32_t rank_top;
    quantile_rank(c.cfg.clip_quantile, BK * D, &kr, &frac, &rank_top);
    uint32_t cmax[S::NC];
    chunk_maxima<S::NC>(v, cmax);
#pragma unroll
    for (int i = 0; i < S::NC; ++i) gmax = max(gmax, cmax[i]);
    fast = clip_candidates<D, BK>(tile, cmax, rank_top, cs, red);
  }
  uint32_t colpk[S::NC];
  if constexpr (KO != 0) row_outliers<D, BK, KO>(v, tile, ko, ocol, oval, colpk);
  __syncthreads();  // the tile, the staged CSR slice and the candidate lists are complete
  if constexpr (KO != 0)
  {
    const bool paged = c.block_table != nullptr;
    int32_t* rp = (is_key ? c.k_rowptr : c.v_rowptr) + (paged ? g * (BK + 1) : bh * (T + 1));
    write_csr<BK, KO>(ocol, oval, rp, (is_key ? c.k_col : c.v_col) + g * BK * ko,
                      (is_key ? c.k_val : c.v_val) + g * BK * ko, paged ? 0 : t0, ko);
  }
  float thr = 0.0f;
  if constexpr (CLIP)
    thr = fast ? clip_from_candidates<BK * D>(cs, red, c.cfg.clip_quantile)
               : clip_from_tile<D, BK>(tile, cs, red, c.cfg.clip_quantile, gmax);
  // the clip's reads of the tile ended at its closing barrier
  if constexpr (KO != 0) mark_outliers<D, BK, KO>(tile, colpk, ko);
  return thr;
}

// ---------------------------------------------------------------- keys kept in fp16
// The R key vectors of the block with the largest squared L2 norm ([TQ] sections 3.2
// and 6.1: importance from the vector's own norm, the important few kept in high
// precision), the norm being the fp64 sum of the exact squares in channel order.  A
// token is kept when fewer than R tokens come before it in (norm descending, token
// ascending).  The kept rows are copied out in ascending token order and marked with
// the outlier mark in the tile, which takes them out of the per-channel statistics and
// gives them code 0.
//
// The sum is taken in parallel (kThreads / BK threads per token, four chains each).
// Every square of a row is an integer multiple of 2^m, m set by the row's smallest
// nonzero exponent, so every partial sum, in any order, is too; while the total stays
// below 2^(m + 53) each of them is an fp64 number, every addition is exact and the
// parallel sum equals the channel-order one bit for bit.  A row past that bound (a
// range of magnitudes beyond 2^26, or a non-finite value) is summed again in channel
// order by one thread.  norm: BK doubles; flag: 256 ints (the waves' kept-token masks,
// the kept tokens in order, the rows summed exactly).
template <int D, int BK>
__device__ __forceinline__ void keep_rows(uint16_t* tile, double* norm, int* flag, const kvq_cache& c, int64_t g) {
  static_assert(BK % kWave == 0 && BK <= 128 && kThreads % BK == 0, "whole waves of tokens, offsets in a byte");
  constexpr int P = D + 8;
  constexpr int TPT = kThreads / BK;  // threads per token
  constexpr int CH = D / TPT;         // channels per thread
  static_assert(CH % 8 == 0 && TPT <= kWave, "16-byte row pieces");
  constexpr int NW = kThreads / kWave;
  const int R = keep_count(c.cfg);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int j = tid / TPT, part = tid % TPT;
  uint32_t* masks = reinterpret_cast<uint32_t*>(flag);  // [NW][2]
  int* order = flag + 2 * NW;                            // [R <= 16]: kept tokens, ascending
  int* exact = flag + 64;                                // [BK]
  {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    uint32_t emin = 31u;  // smallest biased exponent (subnormals as 1) of a nonzero value
    const uint16_t* row = &tile[j * P + part * CH];
#pragma unroll
    for (int d = 0; d < CH; d += 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(row + d);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint16_t hv = (uint16_t)(ws[k >> 1] >> (16 * (k & 1)));
        const double x = (double)h2f(hv);
        acc[k & 3] = __builtin_fma(x, x, acc[k & 3]);
        const uint32_t mag = hv & 0x7fffu;
        emin = min(emin, mag ? max(mag >> 10, 1u) : 31u);
      }
    }
    double sm = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
    for (int o = 1; o < TPT; o <<= 1) {
      sm += __shfl_xor(sm, o, kWave);
      emin = min(emin, (uint32_t)__shfl_xor((int)emin, o, kWave));
    }
    // squares are multiples of 2^(2 e - 50) (e the biased exponent, 1 for subnormals)
    const bool ok = sm < __builtin_ldexp(1.0, 2 * (int)emin - 50 + 53);
    if (part == 0) {
      norm[j] = sm;
      exact[j] = ok ? 1 : 0;
    }
  }
  __syncthreads();
  if (tid < BK && !exact[tid]) {
    double sm = 0.0;
    for (int d = 0; d < D; ++d) {
      const double x = (double)h2f(tile[tid * P + d]);
      sm = __builtin_fma(x, x, sm);  // the square is exact: one rounding per addition
    }
    norm[tid] = sm;
  }
  __syncthreads();
  bool kept;
  {
    const double m = norm[j];
    int before = 0;
    const int k0 = part * (BK / TPT);
#pragma unroll 8
    for (int k = k0; k < k0 + BK / TPT; k += 2) {
      const double2 o = *reinterpret_cast<const double2*>(norm + k);
      before += (o.x > m || (o.x == m && k < j)) ? 1 : 0;
      before += (o.y > m || (o.y == m && k + 1 < j)) ? 1 : 0;
    }
#pragma unroll
    for (int o = 1; o < TPT; o <<= 1) before += __shfl_xor(before, o, kWave);
    kept = part == 0 && before < R;
    const uint64_t bal = __ballot(kept);
    if (lane == 0) {
      masks[2 * wave] = (uint32_t)bal;
      masks[2 * wave + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();
  if (kept) {
    int pos = 0;
    for (int w = 0; w < wave; ++w) pos += __builtin_popcount(masks[2 * w]) + __builtin_popcount(masks[2 * w + 1]);
    const uint64_t mine = (uint64_t)masks[2 * wave] | ((uint64_t)masks[2 * wave + 1] << 32);
    pos += __builtin_popcountll(mine & ((1ull << lane) - 1ull));
    // (finite norms keep exactly R tokens; NaN norms compare false and could claim more)
    if (pos < R) {
      order[pos] = j;
      c.k_keep_idx[g * R + pos] = (uint8_t)j;
    }
  }
  __syncthreads();
  // rows out, 16 bytes a thread, each chunk then marked by the thread that read it
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const uint4 mark = make_uint4(kMarkNaN * 0x10001u, kMarkNaN * 0x10001u, kMarkNaN * 0x10001u, kMarkNaN * 0x10001u);
  for (int e = tid; e < R * CPR; e += kThreads) {
    const int row = e / CPR, ch = e % CPR;
    uint4* src = reinterpret_cast<uint4*>(&tile[order[row] * P + 8 * ch]);
    *reinterpret_cast<uint4*>(c.k_keep_val + (g * R + row) * D + 8 * ch) = *src;
    *src = mark;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- keys
// A key cell is held as its fp16 bits, two elements per register (element q of token
// u in half q % 2 of xw[u][q / 2]), and converted where it is used.
__device__ __forceinline__ float xel(const uint32_t (&xw)[8][4], int u, int q) {
  return h2f((uint16_t)(xw[u][q >> 1] >> (16 * (q & 1))));
}

// Fast codes of a key cell packed into one word per token: element e = 2 (q % 4) + q / 4
// of the cell sits at bits e KB of the word.
template <int KB, bool OUTL, bool CLIP>
__device__ __forceinline__ void key_codes(const uint32_t (&xw)[8][4], const float* zq, const float* rq, const float* aq,
                                          const float* bq, const float* sq, int L, float thr, uint32_t* w) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float cf[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      bool near;
      float qc;
      cf[q] = code_fast_h<OUTL, CLIP>(half_of(xw[u][q >> 1], q & 1), zq[q], rq[q], aq[q], bq[q], near, qc);
      // rare: a quotient this close to a rounding boundary is decided exactly
      if (near) cf[q] = code_near<OUTL, CLIP>(xel(xw, u, q), zq[q], sq[q], qc, (float)L, thr);
    }
    uint32_t wu = 0;
    if constexpr (KB == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wu = put_byte(__builtin_fmaf(cf[4 + i], 16.0f, cf[i]), i, wu);
    } else if constexpr (KB == 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float lo2 = __builtin_fmaf(cf[4 + 2 * k], 4.0f, cf[2 * k]);
        const float hi2 = __builtin_fmaf(cf[5 + 2 * k], 4.0f, cf[2 * k + 1]);
        wu = put_byte(__builtin_fmaf(hi2, 16.0f, lo2), k, wu);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) wu |= (uint32_t)cf[q] << ((2 * (q & 3) + (q >> 2)) * KB);
    }
    w[u] = wu;
    // one token at a time: interleaving the tokens' exact-tie paths costs occupancy
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Cell: 8 tokens x 8 channels, the channels being the rotary pairs 4a..4a+3 and
// D/2+4a..D/2+4a+3, i.e. elements 8a..8a+7 of the packed row (element e holds channel
// e/2 + (e%2) D/2).  Thread tid = a * NTG + tg; the cell's tokens are tg + NTG u, so
// the NTG lanes sharing a channel set form one DPP row and read distinct LDS banks.
// LUTB: 0 for uniform keys (code width from the configuration), else the code width
// of codebook keys.  RET: keys kept in fp16 (uniform keys without outliers or clipping).
template <int D, int BK, int LUTB, int KO, bool CLIP, bool RET>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void quantize_keys_kernel(kvq_cache c, const uint16_t* __restrict__ k_new,
                                                                 int64_t old_len_arg, int64_t n_new, int64_t n_first,
    const int64_t* __restrict__ n_seq) {
  static_assert(!RET || (LUTB == 0 && KO == 0 && !CLIP), "kept keys: uniform keys without outliers or clip");
  constexpr bool OUTL = KO != 0 || RET;  // kept rows carry the outlier mark
  constexpr int P = D + 8;
  constexpr int NTG = BK / 8;
  constexpr int NA = D / 8;
  __shared__ KeySmem<D, BK> sh;
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  // per-sequence lengths: this sequence's own length, its own count of new tokens
  // (n_seq; n_new is then the input's rows per sequence) and the blocks they complete
  const int64_t old_len = c.seq_lens ? seq_len_of(c, b) : old_len_arg;
  // (a device count is clamped to the input's rows, a block to the capacity: a count
  // that disagrees with the host's gives wrong tokens, never an access out of bounds)
  const int64_t n_b = n_seq ? min(max(n_seq[b], (int64_t)0), n_new) : n_new;
  const int64_t n = (c.seq_lens ? old_len / BK : n_first) + blockIdx.x;
  if (n >= (old_len + n_b) / BK || n >= c.cfg.capacity / BK) return;
  const int64_t g = slot_of(c, b, h, n);
  const int64_t T = c.cfg.capacity;
  const int64_t bh = (int64_t)b * c.cfg.kv_heads + h;
  constexpr bool lut = LUTB > 0;
  const int kb = lut ? LUTB : c.cfg.k_bits;
  const int L = (1 << kb) - 1;
  const float Lf = (float)L;

  const float thr =
      prepare_tile<D, BK, KO, CLIP>(sh.u.tile, sh.ocol, sh.oval, sh.clip, sh.red, c, true, k_new, bh, n, g, old_len, n_new);
  __syncthreads();
  if constexpr (RET)  // the clip's candidate lists are free (no clipping here)
    keep_rows<D, BK>(sh.u.tile, reinterpret_cast<double*>(sh.clip.cand),
                     reinterpret_cast<int*>(reinterpret_cast<double*>(sh.clip.cand) + BK), c, g);

  const bool active = NA * NTG == kThreads || tid < NA * NTG;
  const int a = tid / NTG, tg = tid % NTG;
  uint32_t xw[8][4];
  float lo[8], hi[8];
  // per channel min / max over the cell's tokens on packed fp16 pairs (exact)
  uint32_t plo[4] = {kPkPosInf, kPkPosInf, kPkPosInf, kPkPosInf};
  uint32_t phi[4] = {kPkNegInf, kPkNegInf, kPkNegInf, kPkNegInf};
#pragma unroll
  for (int u = 0; u < 8; ++u) xw[u][0] = xw[u][1] = xw[u][2] = xw[u][3] = 0u;
  if (active) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = tg + NTG * u;
      const uint2 wl = *reinterpret_cast<const uint2*>(&sh.u.tile[j * P + 4 * a]);
      const uint2 wh = *reinterpret_cast<const uint2*>(&sh.u.tile[j * P + D / 2 + 4 * a]);
      xw[u][0] = wl.x; xw[u][1] = wl.y; xw[u][2] = wh.x; xw[u][3] = wh.y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        plo[i] = pk_min_h(plo[i], xw[u][i]);
        phi[i] = pk_max_h(phi[i], xw[u][i]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    lo[q] = (float)half_of(plo[q >> 1], q & 1);
    hi[q] = (float)half_of(phi[q >> 1], q & 1);
  }
  __syncthreads();  // the tile is dead from here on; its space holds the outputs
  auto& M = sh.u.out.meta;
  const int chq[8] = {4 * a, 4 * a + 1, 4 * a + 2, 4 * a + 3, D / 2 + 4 * a, D / 2 + 4 * a + 1,
                      D / 2 + 4 * a + 2, D / 2 + 4 * a + 3};
  if constexpr (!lut) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      lo[q] = lanes_min<NTG>(lo[q]);
      hi[q] = lanes_max<NTG>(hi[q]);
    }
    if (CLIP) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        lo[q] = fminf(fmaxf(lo[q], -thr), thr);  // clipping commutes with min and max
        hi[q] = fminf(fmaxf(hi[q], -thr), thr);
      }
    }
    if (active && tg < 8) {
      float l0 = lo[0], h0 = hi[0];
#pragma unroll
      for (int q = 1; q < 8; ++q)
        if (tg == q) { l0 = lo[q]; h0 = hi[q]; }
      uint16_t z16, s16;
      meta_from(l0, h0, L, &z16, &s16);
      const int ch = (tg < 4) ? 4 * a + tg : D / 2 + 4 * a + tg - 4;
      c.k_scale[g * D + ch] = s16;
      c.k_zero[g * D + ch] = z16;
      const float z = h2f(z16), s = h2f(s16), r = recip_or_zero(s);
      float qa, qb;
      quotient_bounds<CLIP>(z, r, Lf, thr, &qa, &qb);
      M.z[ch] = z;
      M.s[ch] = s;
      M.r[ch] = r;
      M.a[ch] = qa;
      M.b[ch] = qb;
    }
  } else {
    for (int ch = tid; ch < D; ch += kThreads) {
      const uint16_t* lt = c.k_lut + ((int64_t)h * D + ch) * (L + 1);
      for (int k = 0; k < L; ++k) sh.u.out.mids[ch * 15 + k] = (h2f(lt[k]) + h2f(lt[k + 1])) * 0.5f;
    }
  }
  __syncthreads();

  const int rk = D * kb / 8;
  const int rkp = rk + 16;
  // the cell is converted again below rather than kept as 64 floats since the statistics
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(xw[u][i]));
  if (active) {
    uint32_t w[8];
    if constexpr (!lut) {
      float zq[8], rq[8], aq[8], bq[8];
      auto ld4 = [&](const float* base, float* dst) {
        const float4 l4 = *reinterpret_cast<const float4*>(base + 4 * a);
        const float4 h4 = *reinterpret_cast<const float4*>(base + D / 2 + 4 * a);
        dst[0] = l4.x; dst[1] = l4.y; dst[2] = l4.z; dst[3] = l4.w;
        dst[4] = h4.x; dst[5] = h4.y; dst[6] = h4.z; dst[7] = h4.w;
      };
      ld4(M.z, zq);
      ld4(M.r, rq);
      if constexpr (CLIP) {
        ld4(M.a, aq);
        ld4(M.b, bq);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) { aq[q] = 0.0f; bq[q] = Lf; }
      }
      float sq[8];
      ld4(M.s, sq);
      if (kb == 4) key_codes<4, OUTL, CLIP>(xw, zq, rq, aq, bq, sq, L, thr, w);
      else if (kb == 2) key_codes<2, OUTL, CLIP>(xw, zq, rq, aq, bq, sq, L, thr, w);
      else key_codes<3, OUTL, CLIP>(xw, zq, rq, aq, bq, sq, L, thr, w);
    } else {
      // code = the number of midpoints below the value (ties to the lower entry)
      constexpr int NM = (1 << (lut ? LUTB : 1)) - 1;
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float md[NM];
#pragma unroll
        for (int k = 0; k < NM; ++k) md[k] = sh.u.out.mids[chq[q] * 15 + k];
        const int e = 2 * (q & 3) + (q >> 2);
        if constexpr (!CLIP) {
          // Unclipped values are fp16 (multiples of 2^-24) and every midpoint is a
          // multiple of 2^-25, so (x - mid) * 2^25 is an integer computed exactly by
          // one FMA: clamped to [0, 1] it is the step [x > mid], with no compare.
#pragma unroll
          for (int k = 0; k < NM; ++k) md[k] *= -33554432.0f;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float d = xel(xw, u, q);
            float st[NM];
#pragma unroll
            for (int k = 0; k < NM; ++k)
              st[k] = __builtin_amdgcn_fmed3f(__builtin_fmaf(d, 33554432.0f, md[k]), 0.0f, 1.0f);
#pragma unroll
            for (int w2 = 1; w2 < NM; w2 *= 2)  // pairwise sum of the steps
#pragma unroll
              for (int k = 0; k + w2 < NM; k += 2 * w2) st[k] += st[k + w2];
            uint32_t cq = (uint32_t)st[0];
            if constexpr (OUTL) cq = (d != d) ? 0u : cq;
            w[u] |= cq << (e * (lut ? LUTB : 1));
          }
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float xv = xel(xw, u, q);
            const float d = fminf(fmaxf(xv, -thr), thr);
            uint32_t cq = 0;
#pragma unroll
            for (int k = 0; k < NM; ++k) cq += d > md[k] ? 1u : 0u;
            if constexpr (OUTL) cq = (xv != xv) ? 0u : cq;
            w[u] |= cq << (e * (lut ? LUTB : 1));
          }
        }
      }
    }
    // the cell's kb bytes of each token row
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uint8_t* dst = &sh.u.out.krow[(tg + NTG * u) * rkp + a * kb];
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
  uint8_t* out = static_cast<uint8_t*>(c.k_codes) + g * BK * rk;
  if (rk % 16 == 0) {
    const int per_row = rk / 16;
    for (int idx = tid; idx < BK * per_row; idx += kThreads) {
      const int j = idx / per_row, p = idx % per_row;
      reinterpret_cast<uint4*>(out)[idx] = *reinterpret_cast<const uint4*>(&sh.u.out.krow[j * rkp + p * 16]);
    }
  } else {
    const int per_row = rk / 8;
    for (int idx = tid; idx < BK * per_row; idx += kThreads) {
      const int j = idx / per_row, p = idx % per_row;
      reinterpret_cast<uint2*>(out)[idx] = *reinterpret_cast<const uint2*>(&sh.u.out.krow[j * rkp + p * 8]);
    }
  }
}

// ---------------------------------------------------------------- values
// Cell: TPW = 32/VB consecutive tokens x CW channels, so that each of its CW channels
// yields one packed word.  Thread tid = tg * NCC + cc: the lanes of one value group
// are consecutive, and the row statistics reduce across them.
// Row statistics over the lpg lanes of a value group, for all TPW tokens of a cell.
template <int TPW>
__device__ __forceinline__ void vgroup_minmax(float* lo, float* hi, int lpg) {
  if (lpg >= 2) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) { lo[u] = min_x1(lo[u]); hi[u] = max_x1(hi[u]); }
  }
  if (lpg >= 4) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) { lo[u] = min_x2(lo[u]); hi[u] = max_x2(hi[u]); }
  }
  if (lpg >= 8) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) { lo[u] = min_hm(lo[u]); hi[u] = max_hm(hi[u]); }
  }
  if (lpg >= 16) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) { lo[u] = min_rm(lo[u]); hi[u] = max_rm(hi[u]); }
  }
  if (lpg >= 32) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      lo[u] = fminf(lo[u], __shfl_xor(lo[u], 16, kWave));
      hi[u] = fmaxf(hi[u], __shfl_xor(hi[u], 16, kWave));
    }
  }
}

template <int D, int BK, int VB, int KO, bool CLIP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void quantize_values_kernel(kvq_cache c, const uint16_t* __restrict__ v_new,
                                                                   int64_t old_len_arg, int64_t n_new, int64_t n_first,
    const int64_t* __restrict__ n_seq) {
  constexpr bool OUTL = KO != 0;
  constexpr int P = D + 8;
  constexpr int TPW = 32 / VB;
  constexpr int CW = VB == 4 ? 8 : 4;
  constexpr int NCC = D / CW;
  constexpr int NTG = BK / TPW;
  __shared__ ValueSmem<D, BK> sh;
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  // per-sequence lengths: this sequence's own length, its own count of new tokens
  // (n_seq; n_new is then the input's rows per sequence) and the blocks they complete
  const int64_t old_len = c.seq_lens ? seq_len_of(c, b) : old_len_arg;
  // (a device count is clamped to the input's rows, a block to the capacity: a count
  // that disagrees with the host's gives wrong tokens, never an access out of bounds)
  const int64_t n_b = n_seq ? min(max(n_seq[b], (int64_t)0), n_new) : n_new;
  const int64_t n = (c.seq_lens ? old_len / BK : n_first) + blockIdx.x;
  if (n >= (old_len + n_b) / BK || n >= c.cfg.capacity / BK) return;
  const int64_t g = slot_of(c, b, h, n);
  const int64_t bh = (int64_t)b * c.cfg.kv_heads + h;
  const int L = (1 << VB) - 1;
  const float Lf = (float)L;
  const int G = c.cfg.v_group, ng = D / G;
  const int lpg = G / CW;

  const float thr =
      prepare_tile<D, BK, KO, CLIP>(sh.u.tile, sh.ocol, sh.oval, sh.clip, sh.red, c, false, v_new, bh, n, g, old_len, n_new);
  __syncthreads();

  const bool active = NCC * NTG == kThreads || tid < NCC * NTG;
  const int tg = tid / NCC, cc = tid % NCC;
  const int ch0 = cc * CW, grp = ch0 / G;
  // the cell as fp16 pairs (channel q of token u in half q % 2 of xr[u][q / 2]); row
  // min / max over the cell's channels on packed pairs (exact), then over the lanes
  uint32_t xr[TPW][CW / 2];
  float lo[TPW], hi[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    uint32_t mn = kPkPosInf, mx = kPkNegInf;
#pragma unroll
    for (int i = 0; i < CW / 2; ++i) xr[u][i] = 0u;
    if (active) {
      const int j = TPW * tg + u;
      if constexpr (CW == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sh.u.tile[j * P + ch0]);
        xr[u][0] = v.x; xr[u][1] = v.y; xr[u][2] = v.z; xr[u][3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(&sh.u.tile[j * P + ch0]);
        xr[u][0] = v.x; xr[u][1] = v.y;
      }
      if constexpr (CW == 8) {
        mn = pk_min_h(pk_min_h(xr[u][0], xr[u][1]), pk_min_h(xr[u][2], xr[u][3]));
        mx = pk_max_h(pk_max_h(xr[u][0], xr[u][1]), pk_max_h(xr[u][2], xr[u][3]));
      } else {
        mn = pk_min_h(xr[u][0], xr[u][1]);
        mx = pk_max_h(xr[u][0], xr[u][1]);
      }
    }
    lo[u] = fminf((float)half_of(mn, 0), (float)half_of(mn, 1));
    hi[u] = fmaxf((float)half_of(mx, 0), (float)half_of(mx, 1));
  }
  vgroup_minmax<TPW>(lo, hi, lpg);
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (CLIP) {
      lo[u] = fminf(fmaxf(lo[u], -thr), thr);
      hi[u] = fminf(fmaxf(hi[u], -thr), thr);
    }
  }
  __syncthreads();  // the tile is dead from here on; its space holds the metadata
  auto& M = sh.u.meta;
  if (active) {
    const int gi = cc % lpg;
    for (int u0 = 0; u0 < TPW; u0 += lpg) {
      const int uu = u0 + gi;
      if (uu < TPW) {
        float l0 = lo[0], h0 = hi[0];
#pragma unroll
        for (int u = 1; u < TPW; ++u)
          if (uu == u) { l0 = lo[u]; h0 = hi[u]; }
        uint16_t z16, s16;
        meta_from(l0, h0, L, &z16, &s16);
        const int j = TPW * tg + uu;
        c.v_scale[(g * BK + j) * ng + grp] = s16;
        c.v_zero[(g * BK + j) * ng + grp] = z16;
        const float z = h2f(z16), s = h2f(s16), r = recip_or_zero(s);
        float qa, qb;
        quotient_bounds<CLIP>(z, r, Lf, thr, &qa, &qb);
        const int m = grp * BK + j;
        M.z[m] = z;
        M.s[m] = s;
        M.r[m] = r;
        M.a[m] = qa;
        M.b[m] = qb;
      }
    }
  }
  __syncthreads();
  if (active) {
    const int m0 = grp * BK + TPW * tg;
    float zu[TPW], ru[TPW], au[TPW], bu[TPW];
    auto ldt = [&](const float* base, float* dst) {
#pragma unroll
      for (int u = 0; u < TPW; u += 4) {
        const float4 f = *reinterpret_cast<const float4*>(base + m0 + u);
        dst[u] = f.x; dst[u + 1] = f.y; dst[u + 2] = f.z; dst[u + 3] = f.w;
      }
    };
    ldt(M.z, zu);
    ldt(M.r, ru);
    if constexpr (CLIP) {
      ldt(M.a, au);
      ldt(M.b, bu);
    } else {
#pragma unroll
      for (int u = 0; u < TPW; ++u) { au[u] = 0.0f; bu[u] = Lf; }
    }
    uint32_t w[CW];
#pragma unroll
    for (int q = 0; q < CW; ++q) w[q] = 0;
    float su[TPW];
    ldt(M.s, su);
    // token u of the word sits at bits u VB: 4-bit codes pair into bytes, 2-bit
    // codes come in fours
    constexpr int TPB = 8 / VB;  // tokens per byte
#pragma unroll
    for (int k = 0; k < TPW / TPB; ++k) {
      float cf[TPB][CW];
      bool anynear = false;
#pragma unroll
      for (int t = 0; t < TPB; ++t)
#pragma unroll
        for (int q = 0; q < CW; ++q) {
          const int u = k * TPB + t;
          bool near;
          float qc;
          cf[t][q] = code_fast_h<OUTL, CLIP>(half_of(xr[u][q >> 1], q & 1), zu[u], ru[u], au[u], bu[u], near, qc);
          anynear = anynear || near;
        }
      // rare: a quotient this close to a rounding boundary is decided exactly (the fast
      // quotient is recomputed there, bit for bit the same)
      if (anynear) {
#pragma unroll
        for (int t = 0; t < TPB; ++t)
#pragma unroll
          for (int q = 0; q < CW; ++q) {
            const int u = k * TPB + t;
            const _Float16 hq = half_of(xr[u][q >> 1], q & 1);
            bool near;
            float qc;
            (void)code_fast_h<OUTL, CLIP>(hq, zu[u], ru[u], au[u], bu[u], near, qc);
            if (near) cf[t][q] = code_near<OUTL, CLIP>((float)hq, zu[u], su[u], qc, (float)L, thr);
          }
      }
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        float byte = cf[TPB - 1][q];
#pragma unroll
        for (int t = TPB - 2; t >= 0; --t) byte = __builtin_fmaf(byte, (float)(1 << VB), cf[t][q]);
        w[q] = put_byte(byte, k, w[q]);
      }
    }
    uint32_t* out = static_cast<uint32_t*>(c.v_codes) + (g * (BK / TPW) + tg) * D + ch0;
    reinterpret_cast<uint4*>(out)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    if constexpr (CW == 8) reinterpret_cast<uint4*>(out)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

}  // namespace qb
}  // namespace kvq
