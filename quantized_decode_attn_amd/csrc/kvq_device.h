// kvq_device.h -- device helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kWave = 64;

// ---------------------------------------------------------------- fp16 helpers
// Conversions use the hardware v_cvt_f32_f16 / v_cvt_f16_f32 (round to nearest even).
__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h_rn(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

__device__ __forceinline__ uint16_t h_step_down(uint16_t h) {
  if ((h & 0x7fff) == 0) return 0x8001;
  return (h & 0x8000) ? (uint16_t)(h + 1) : (uint16_t)(h - 1);
}
__device__ __forceinline__ uint16_t h_step_up(uint16_t h) {
  if ((h & 0x7fff) == 0) return 0x0001;
  return (h & 0x8000) ? (uint16_t)(h - 1) : (uint16_t)(h + 1);
}
// Largest fp16 not above v, and smallest fp16 not below v (directed rounding done
// as round-to-nearest followed by a one-step correction of the bit pattern).
__device__ __forceinline__ uint16_t f2h_rd(float v) {
  uint16_t h = f2h_rn(v);
  return h2f(h) > v ? h_step_down(h) : h;
}
__device__ __forceinline__ uint16_t f2h_ru(float v) {
  uint16_t h = f2h_rn(v);
  return h2f(h) < v ? h_step_up(h) : h;
}

// ---------------------------------------------------------------- cross-lane
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror: lane i <-> 7-i within 8
constexpr int kDppRowMirror = 0x140;    // row_mirror: lane i <-> 15-i within 16

// Sum over aligned groups of N lanes (N in {1,2,4,8,16}); every lane of the group
// receives the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp_f<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f<kDppRowMirror>(v);
  return v;
}

// Minimum / maximum over aligned groups of N lanes (N in {1,2,4,8,16}), delivered to
// every lane of the group.  fminf/fmaxf return the other operand for a quiet NaN.
template <int N>
__device__ __forceinline__ float group_min(float v) {
  if constexpr (N >= 2) v = fminf(v, dpp_f<kDppQuadXor1>(v));
  if constexpr (N >= 4) v = fminf(v, dpp_f<kDppQuadXor2>(v));
  if constexpr (N >= 8) v = fminf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fminf(v, dpp_f<kDppRowMirror>(v));
  return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  return v;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
// Unsigned maximum over the 16 lanes of a DPP row.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u<kDppQuadXor1>(v));
  v = max(v, dpp_u<kDppQuadXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppRowMirror>(v));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Wave-local ordering point for LDS traffic exchanged between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int kout_of(const kvq_config& c) {
  return c.outlier_pct > 0 ? (c.outlier_pct * c.head_dim + 99) / 100 : 0;
}

// OCP FP8 E4M3 ("e4m3fn": 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
// S.1111.111 = NaN, largest finite 448), the element format of an FP8 cache ([UQ]
// section 2.1).  fp16 -> E4M3 rounds to nearest, ties to even, in integer arithmetic on
// the fp16 fields: the significand (1024 + m, or m for a subnormal) is shifted right to
// the E4M3 unit of the value's binade (2^(E-3), at least 2^-9); magnitudes past 448
// (infinities included) saturate to +-448, NaN stays NaN.
__host__ __device__ __forceinline__ uint32_t f16_to_e4m3(uint32_t h) {
  const uint32_t sign = (h >> 8) & 0x80u;
  const uint32_t mag = h & 0x7FFFu;
  if (mag > 0x7C00u) return sign | 0x7Fu;
  if (mag == 0x7C00u) return sign | 0x7Eu;
  const int e16 = (int)(mag >> 10);
  const uint32_t sig = e16 ? (0x400u | (mag & 0x3FFu)) : (mag & 0x3FFu);  // value = sig 2^(max(e16,1)-25)
  int ex = (e16 ? e16 : 1) - 15;                                          // binade of a normal fp16
  if (ex < -6) ex = -6;
  const int sh = ex + 22 - (e16 ? e16 : 1);                               // >= 7
  uint32_t q = 0u;
  if (sh < 32) {
    const uint32_t keep = sig >> sh, rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
    q = keep + ((rem > half || (rem == half && (keep & 1u))) ? 1u : 0u);
  }
  if (q >= 16u) {  // rounded up into the next binade
    q >>= 1;
    ex += 1;
  }
  if (ex > 8 || (ex == 8 && q > 14u)) return sign | 0x7Eu;  // above 448
  if (ex == -6 && q < 8u) return sign | q;                   // subnormal (or zero)
  return sign | ((uint32_t)(ex + 7) << 3) | (q - 8u);
}
__host__ __device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 0u) v = (float)m * 0x1p-9f;
  else v = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));  // 2^(e-7) (1 + m/8)
  if (e == 15u && m == 7u) v = __builtin_nanf("");
  return (b & 0x80u) ? -v : v;
}

// Tokens of sequence b: its own length in a paged cache (clamped into [0, capacity]),
// else the cache's one length.
__device__ __forceinline__ int64_t seq_len_of(const kvq_cache& c, int64_t b) {
  if (!c.seq_lens) return c.length;
  const int64_t L = c.seq_lens[b];
  return L < 0 ? 0 : (L > c.cfg.capacity ? (int64_t)c.cfg.capacity : L);
}

// The slot of block n of (b, kv head h): every per-block buffer is an array of slots.
// Dense layout: (b * kv_heads + h) * (T / Bk) + n.  Paged: the physical block of
// (b, n) from the table (clamped into the pool) times kv_heads, plus h.
__device__ __forceinline__ int64_t slot_of(const kvq_cache& c, int64_t b, int64_t h, int64_t n) {
  const int64_t nb = c.cfg.capacity / c.cfg.k_block;
  if (!c.block_table) return (b * c.cfg.kv_heads + h) * nb + n;
  int64_t p = c.block_table[b * nb + n];
  p = p < 0 ? 0 : (p >= c.num_blocks ? (int64_t)c.num_blocks - 1 : p);
  return p * c.cfg.kv_heads + h;
}

// The slots of one (b, kv head), with the division by the block size done once: the
// slot of block 0 in the dense layout, or the sequence's row of the block table.
struct SlotRow {
  int64_t base;
  const int32_t* row;
  int64_t last;  // num_blocks - 1
  int64_t H, h;
};
__device__ __forceinline__ SlotRow slot_row(const kvq_cache& c, int64_t b, int64_t h) {
  const int64_t nb = c.cfg.capacity / c.cfg.k_block;
  SlotRow s;
  s.base = (b * c.cfg.kv_heads + h) * nb;
  s.row = c.block_table ? c.block_table + b * nb : nullptr;
  s.last = (int64_t)c.num_blocks - 1;
  s.H = c.cfg.kv_heads;
  s.h = h;
  return s;
}
// Block n's slot (slot_of); PG false: the dense layout, known at compile time.
template <bool PG>
__device__ __forceinline__ int64_t slot_at(const SlotRow& s, int64_t n) {
  if constexpr (PG) {
    if (s.row) {
      int64_t p = s.row[n];
      p = p < 0 ? 0 : (p > s.last ? s.last : p);
      return p * s.H + s.h;
    }
  }
  return s.base + n;
}

// The same with the layout fixed at compile time: PG (per-sequence lengths, dense or
// paged slots) or the dense layout with one length, whose kernels then carry no
// paging code at all.
template <bool PG>
__device__ __forceinline__ int64_t seq_len_t(const kvq_cache& c, int64_t b) {
  if constexpr (PG) return seq_len_of(c, b);
  else return c.length;
}
template <bool PG>
__device__ __forceinline__ int64_t slot_t(const kvq_cache& c, int64_t b, int64_t h, int64_t n) {
  if constexpr (PG) return slot_of(c, b, h, n);
  else return (b * c.cfg.kv_heads + h) * (c.cfg.capacity / c.cfg.k_block) + n;
}

}  // namespace kvq
