// decode_common.h -- pieces shared by the decode kernels over uniform 2/4-bit caches:
// the per-lane work shape, the packed-code unpacking, the register block of one
// (b, kv-head, block) and its loaders, and the cross-lane reductions.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace dcm {

constexpr float kLog2e = 1.4426950408889634f;

// Work items of a cache with per-sequence lengths: every item of sequence b costs about
// len_b / S blocks.  The host sorts the sequences by their host lengths, longest first,
// and the waves take the items in that order in a snake: wave p takes item
// r * nw + p in even rounds r and r * nw + nw - 1 - p in odd ones, so that a wave with a
// long item in one round gets a short one in the next.  n == 0: natural order.
constexpr int kOrderMax = 1024;
struct SeqOrder {
  int32_t n;
  uint16_t b[kOrderMax];
};
inline SeqOrder seq_order(const kvq_cache& c) {
  SeqOrder o;
  o.n = 0;
  const int B = c.cfg.batch;
  if (!c.seq_lens_host || B > kOrderMax) return o;
  for (int b = 0; b < B; ++b) o.b[b] = (uint16_t)b;
  // insertion sort, longest first, ties in sequence order (B is small)
  for (int i = 1; i < B; ++i) {
    const uint16_t x = o.b[i];
    const int64_t lx = c.seq_lens_host[x];
    int j = i - 1;
    while (j >= 0 && c.seq_lens_host[o.b[j]] < lx) {
      o.b[j + 1] = o.b[j];
      --j;
    }
    o.b[j + 1] = x;
  }
  o.n = B;
  return o;
}
__device__ __forceinline__ int64_t snake_item(int64_t r, int64_t p, int64_t nw) {
  return r * nw + ((r & 1) ? nw - 1 - p : p);
}
// The natural index of the k-th item in length order (per_seq items per sequence).
__device__ __forceinline__ int64_t ordered_item(const SeqOrder& ord, int64_t k, int64_t per_seq) {
  const int64_t qs = k / per_seq, rest = k - qs * per_seq;
  return (ord.n ? (int64_t)ord.b[qs] : qs) * per_seq + rest;
}

template <int D, int BK, int KB, int VB, int PPL_ = 8>
struct MShape {
  static constexpr int HALF = D / 2;
  static constexpr int PPL = PPL_;               // rotary pairs per lane
  static constexpr int LPT = HALF / PPL;         // lanes per key token
  static constexpr int TPI = kWave / LPT;        // key tokens per iteration
  static constexpr int NIT = BK / TPI;           // iterations per block
  static constexpr int KW = (2 * PPL * KB + 31) / 32;  // code dwords per lane per token (3-bit: 48 bits in 2)
  static constexpr int RK = D * KB / 8;          // key row bytes
  static constexpr int TPW = 32 / VB;            // tokens per value word
  static constexpr int WPB = (BK / TPW) * D;     // value words per block
  static constexpr int NVI = WPB / 256;          // 16-byte value loads per lane per block
  // LDS copy of the rotary table: a row holds the (cos, sin) of one token offset for
  // every pair, as 16-byte chunks ordered [chunk q4 of a lane][lane of the token], so
  // the LPT lanes of a token read consecutive chunks; the pitch D + D/4 puts the
  // tokens read together by one instruction into distinct bank groups as well
  static constexpr int TPITCH = D + D / 4;       // floats per rotary-table row
  static constexpr int CHL = D / 4;              // lanes owning distinct value channels
  // float offset of pair i's (cos, sin) in a row
  static __host__ __device__ constexpr int tab_off(int i) {
    return 4 * (LPT * ((i % PPL) / 2) + i / PPL) + 2 * (i % 2);
  }
};

typedef float f2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f2v cvt_lo(uint32_t x) { return __builtin_amdgcn_cvt_pk_f32_fp8(x, false); }
__device__ __forceinline__ f2v cvt_hi(uint32_t x) { return __builtin_amdgcn_cvt_pk_f32_fp8(x, true); }

// Codes of one lane's 8 rotary pairs as floats (times the fp8 unit).
template <int KB, int KW>
__device__ __forceinline__ void unpack_pairs(const uint32_t (&w)[KW], float (&ca)[8], float (&cb)[8]) {
  if constexpr (KB == 4) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t lo = w[d] & 0x0F0F0F0Fu, hi = (w[d] >> 4) & 0x0F0F0F0Fu;
      const f2v a01 = cvt_lo(lo), a23 = cvt_hi(lo), b01 = cvt_lo(hi), b23 = cvt_hi(hi);
      ca[4 * d] = a01.x; ca[4 * d + 1] = a01.y; ca[4 * d + 2] = a23.x; ca[4 * d + 3] = a23.y;
      cb[4 * d] = b01.x; cb[4 * d + 1] = b01.y; cb[4 * d + 2] = b23.x; cb[4 * d + 3] = b23.y;
    }
  } else {
    const uint32_t x0 = w[0] & 0x03030303u, x1 = (w[0] >> 2) & 0x03030303u;
    const uint32_t x2 = (w[0] >> 4) & 0x03030303u, x3 = (w[0] >> 6) & 0x03030303u;
    f2v t;
    t = cvt_lo(x0); ca[0] = t.x; ca[2] = t.y;
    t = cvt_hi(x0); ca[4] = t.x; ca[6] = t.y;
    t = cvt_lo(x2); ca[1] = t.x; ca[3] = t.y;
    t = cvt_hi(x2); ca[5] = t.x; ca[7] = t.y;
    t = cvt_lo(x1); cb[0] = t.x; cb[2] = t.y;
    t = cvt_hi(x1); cb[4] = t.x; cb[6] = t.y;
    t = cvt_lo(x3); cb[1] = t.x; cb[3] = t.y;
    t = cvt_hi(x3); cb[5] = t.x; cb[7] = t.y;
  }
}

// 4-bit codes of one lane's 8 rotary pairs as exact fp16 subnormals, for FMAs that read
// them with v_fma_mix_f32 (no conversion instruction): a nibble masked into bits 0-3
// of a 16-bit half is the fp16 value c * 2^-24, one in bits 4-7 is c * 2^-20.  Byte b
// of dword d holds pair 4 d + b (code_a low, code_b high); bytes 0 and 2 are read in
// place, bytes 1 and 3 after one shift, so 8 codes cost 5 bit operations.  The caller
// scales code_a coefficients by 2^24 and code_b coefficients by 2^20.
typedef _Float16 h2t __attribute__((ext_vector_type(2)));
template <int KW>
__device__ __forceinline__ void unpack4_f16(const uint32_t (&w)[KW], float (&ca)[8], float (&cb)[8]) {
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t t = w[d] >> 8;
    const h2t a02 = __builtin_bit_cast(h2t, w[d] & 0x000F000Fu), b02 = __builtin_bit_cast(h2t, w[d] & 0x00F000F0u);
    const h2t a13 = __builtin_bit_cast(h2t, t & 0x000F000Fu), b13 = __builtin_bit_cast(h2t, t & 0x00F000F0u);
    ca[4 * d] = (float)a02.x; ca[4 * d + 2] = (float)a02.y; ca[4 * d + 1] = (float)a13.x; ca[4 * d + 3] = (float)a13.y;
    cb[4 * d] = (float)b02.x; cb[4 * d + 2] = (float)b02.y; cb[4 * d + 1] = (float)b13.x; cb[4 * d + 3] = (float)b13.y;
  }
}

// All global data of one block that a wave needs, held in registers.
// KS key slots: a whole block (the default) or half of one, refilled twice per block;
// PPL rotary pairs per lane.
template <int D, int BK, int KB, int VB, int KS = MShape<D, BK, KB, VB>::NIT, int PPL = 8>
struct BlockRegs {
  using Sh = MShape<D, BK, KB, VB, PPL>;
  uint32_t k[KS][Sh::KW];
  uint4 v[Sh::NVI];
  uint16_t kmeta[4];      // lane i < D/2: scale[i], scale[i+D/2], zero[i], zero[i+D/2]
  float eb_c, eb_s;       // lane i < D/2: cos/sin(n*Bk*f_i)
  uint16_t vs[4], vz[4];  // value scale/zero of elements lane + 64*k
  uint32_t kcol, vcol;    // outlier CSR slice of the block (bytes lane*4..)
  uint2 kval, vval;       // (bytes lane*8..)
};

// Loaders of the pieces of one block, each into its own register slot, so that a
// slot can be refilled with the next block as soon as it has been consumed.  Every
// address is a wave-uniform block base plus a 32-bit lane offset.  A block is named by
// its slot g (slot_of: the same in the dense and the paged layout); the rotary block
// base takes its position n.
template <int D, int BK, int KB, int VB>
__device__ __forceinline__ const uint8_t* k_block(const kvq_cache& c, int64_t g) {
  using Sh = MShape<D, BK, KB, VB>;
  return static_cast<const uint8_t*>(c.k_codes) + g * BK * Sh::RK;
}
template <int D, int BK, int KB, int VB>
__device__ __forceinline__ const uint8_t* v_block(const kvq_cache& c, int64_t g) {
  using Sh = MShape<D, BK, KB, VB>;
  return reinterpret_cast<const uint8_t*>(static_cast<const uint32_t*>(c.v_codes) + g * (BK / Sh::TPW) * D);
}

// Key codes of iteration `it` of a block into slot `slot`.
template <int D, int BK, int KB, int VB, int KS, int PPL>
__device__ __forceinline__ void load_k_slot(BlockRegs<D, BK, KB, VB, KS, PPL>& R, int slot, int it,
                                            const uint8_t* kblk, uint32_t koff) {
  using Sh = MShape<D, BK, KB, VB, PPL>;
  const uint8_t* kc = kblk + koff + it * (Sh::TPI * Sh::RK);
  static_assert(Sh::KW >= 1, "a lane reads at least one dword of codes per token");
  // codes are read once: non-temporal loads
  if constexpr (Sh::KW == 2) {
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
    const u2v x = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(kc));
    R.k[slot][0] = x.x;
    R.k[slot][1] = x.y;
  } else {
    R.k[slot][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kc));
  }
}
template <int D, int BK, int KB, int VB>
__device__ __forceinline__ void load_k(BlockRegs<D, BK, KB, VB>& R, int it, const uint8_t* kblk, uint32_t koff) {
  load_k_slot(R, it, it, kblk, koff);
}

template <int D, int BK, int KB, int VB, int KS, int PPL>
__device__ __forceinline__ void load_v(BlockRegs<D, BK, KB, VB, KS, PPL>& R, int i, const uint8_t* vblk, int lane) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const u4v x = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(vblk + (uint32_t)(i * 64 + lane) * 16u));
  R.v[i] = make_uint4(x.x, x.y, x.z, x.w);
}

template <int D, int BK, int KB, int VB, int KS, int PPL>
__device__ __forceinline__ void load_kmeta(BlockRegs<D, BK, KB, VB, KS, PPL>& R, const kvq_cache& c, int64_t g, int64_t n,
                                           int lane, int ko) {
  using Sh = MShape<D, BK, KB, VB>;
  if (lane < Sh::HALF) {
    const int64_t m = g * D;
    const uint16_t* ks = c.k_scale + m;
    const uint16_t* kz = c.k_zero + m;
    R.kmeta[0] = ks[lane];
    R.kmeta[1] = ks[lane + Sh::HALF];
    R.kmeta[2] = kz[lane];
    R.kmeta[3] = kz[lane + Sh::HALF];
    const float2 eb = reinterpret_cast<const float2*>(c.rope + (int64_t)BK * D + n * D)[lane];
    R.eb_c = eb.x;
    R.eb_s = eb.y;
  }
  if (ko > 0) {
    const int nb = BK * ko;
    const int64_t e0 = g * BK * ko;
    if (lane * 4 < nb) {
      R.kcol = reinterpret_cast<const uint32_t*>(c.k_col + e0)[lane];
      R.vcol = reinterpret_cast<const uint32_t*>(c.v_col + e0)[lane];
      R.kval = reinterpret_cast<const uint2*>(c.k_val + e0)[lane];
      R.vval = reinterpret_cast<const uint2*>(c.v_val + e0)[lane];
    }
  }
}

// Outlier CSR slice of block n: entries 4*lane .. 4*lane+3 (columns and values of
// the key and the value outliers); BK * ko <= 256.
template <int D, int BK, int KB, int VB, int KS, int PPL>
__device__ __forceinline__ void load_csr(BlockRegs<D, BK, KB, VB, KS, PPL>& R, const kvq_cache& c, int64_t g,
                                         int lane, int ko) {
  const int nb = BK * ko;
  const int64_t e0 = g * BK * ko;
  if (lane * 4 < nb) {
    R.kcol = reinterpret_cast<const uint32_t*>(c.k_col + e0)[lane];
    R.vcol = reinterpret_cast<const uint32_t*>(c.v_col + e0)[lane];
    R.kval = reinterpret_cast<const uint2*>(c.k_val + e0)[lane];
    R.vval = reinterpret_cast<const uint2*>(c.v_val + e0)[lane];
  }
}

template <int D, int BK, int KB, int VB, int KS, int PPL>
__device__ __forceinline__ void load_vmeta(BlockRegs<D, BK, KB, VB, KS, PPL>& R, const kvq_cache& c, int64_t g,
                                           int lane, int ng) {
  const int ne = BK * ng;
  const int64_t m0 = g * BK * ng;
  const uint16_t* vs = c.v_scale + m0;
  const uint16_t* vz = c.v_zero + m0;
  // every load is issued (an element past the block's ne reads element 0, and its
  // value goes unused): with no load under a branch, the compiler can keep the next
  // block's loads in flight across the block loop instead of draining them
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = lane + 64 * k;
    const bool in = e < ne;
    const int grp = in ? e / BK : 0, t = in ? e % BK : 0;
    const uint32_t m = (uint32_t)(t * ng + grp);
    R.vs[k] = vs[m];
    R.vz[k] = vz[m];
  }
}

// Sum over aligned groups of N lanes (N in {2, 4, 8}), one DPP add per step.
template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  if constexpr (N >= 2) asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "+v"(v));
  if constexpr (N >= 4) asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "+v"(v));
  if constexpr (N >= 8) asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf" : "+v"(v));
  static_assert(N <= 8, "groups of at most 8 lanes");
  return v;
}

// Four independent sums over aligned groups of N lanes (N in {4, 8}).  The DPP steps
// of the four values are interleaved, so each DPP read of a register comes at least
// three instructions after the write that produced it (the hazard needs two wait
// states); one s_nop covers the writes made before the block.
template <int N>
__device__ __forceinline__ void lanes_sum4(float (&v)[4]) {
  static_assert(N == 4 || N == 8, "groups of 4 or 8 lanes");
#define KVQ_DPP4(ctl)                                                          \
  "v_add_f32_dpp %0, %0, %0 " ctl " row_mask:0xf bank_mask:0xf\n\t"           \
  "v_add_f32_dpp %1, %1, %1 " ctl " row_mask:0xf bank_mask:0xf\n\t"           \
  "v_add_f32_dpp %2, %2, %2 " ctl " row_mask:0xf bank_mask:0xf\n\t"           \
  "v_add_f32_dpp %3, %3, %3 " ctl " row_mask:0xf bank_mask:0xf\n\t"
  if constexpr (N == 8)
    asm("s_nop 1\n\t" KVQ_DPP4("quad_perm:[1,0,3,2]") KVQ_DPP4("quad_perm:[2,3,0,1]") KVQ_DPP4("row_half_mirror")
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
  else
    asm("s_nop 1\n\t" KVQ_DPP4("quad_perm:[1,0,3,2]") KVQ_DPP4("quad_perm:[2,3,0,1]")
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
#undef KVQ_DPP4
}

// Maximum over the wave, returned wave-uniform: row maxima by DPP, then the
// row_bcast steps carry them to lane 63.  Operands are scores or weights (never
// signaling NaNs), so no quieting is needed around the cross-lane reads.
__device__ __forceinline__ float wave_max_uniform(float v) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf" : "+v"(v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over the wave, returned wave-uniform (same DPP pattern as wave_max_uniform: every
// lane of a row holds the row sum after the mirrors, the row_bcast steps add the rows).
__device__ __forceinline__ float wave_sum_uniform(float v) {
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf" : "+v"(v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}


// Outlier CSR entries (KO = 1 or 2 per token) of the lane's tokens lane + 64 k
// (k < BK / 64) of a block: a token's columns in one u8/u16, its values in one u16/u32,
// entry q at byte q (columns) and half-word q (values).
struct CsrTok {
  uint32_t kc[2], kv[2], vc[2], vv[2];
};
template <int BK, int KO>
__device__ __forceinline__ void load_csr_tok(CsrTok& C, const kvq_cache& c, int64_t g, int lane) {
  static_assert(KO == 1 || KO == 2, "one or two outliers per vector");
  const int64_t e0 = g * BK * KO;
#pragma unroll
  for (int k = 0; k < BK / kWave; ++k) {
    const int t = lane + kWave * k;
    // outlier entries are read once: non-temporal loads
    if constexpr (KO == 2) {
      C.kc[k] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(c.k_col + e0 + 2 * t));
      C.vc[k] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(c.v_col + e0 + 2 * t));
      C.kv[k] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c.k_val + e0 + 2 * t));
      C.vv[k] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c.v_val + e0 + 2 * t));
    } else {
      C.kc[k] = __builtin_nontemporal_load(c.k_col + e0 + t);
      C.vc[k] = __builtin_nontemporal_load(c.v_col + e0 + t);
      C.kv[k] = __builtin_nontemporal_load(c.k_val + e0 + t);
      C.vv[k] = __builtin_nontemporal_load(c.v_val + e0 + t);
    }
  }
}

// Value-outlier corrections p * (x - zero) are scattered into an LDS channel array with
// integer adds (ds_add_u32 runs several times faster than ds_add_f32): every block's
// corrections of one head are fixed point with the power-of-two scale 2^sh chosen from
// the sum A < 2^e of |correction| over the whole wave, sh = 30 - e.  Every channel sum,
// and every term, then stays below 2^30 in magnitude, and the rounding error is at most
// 2^-31 2^e <= 2^-30 A per term: at most BK 2^-30 A per channel and block (a channel
// takes at most one term per token), i.e. fp32-class relative to the corrections' total.
__device__ __forceinline__ int vcorr_shift(float abs_sum_uniform) {
  return 30 - __builtin_amdgcn_frexp_expf(abs_sum_uniform);
}
__device__ __forceinline__ int vcorr_fixed(float c, int sh) {
  return (int)__builtin_rintf(__builtin_amdgcn_ldexpf(c, sh));
}

// Adds one head's value-outlier corrections accumulated in LDS (D fixed-point ints at
// scale 2^sh) to the lane's channels 4*lane .. 4*lane+3 and clears them.
template <int D>
__device__ __forceinline__ void merge_vcorr(int* VCI, int sh, float (&acc)[4], int lane) {
  if (lane < D / 4) {
    int4* pc = reinterpret_cast<int4*>(VCI + 4 * lane);
    const int4 v = *pc;
    acc[0] += __builtin_amdgcn_ldexpf((float)v.x, -sh);
    acc[1] += __builtin_amdgcn_ldexpf((float)v.y, -sh);
    acc[2] += __builtin_amdgcn_ldexpf((float)v.z, -sh);
    acc[3] += __builtin_amdgcn_ldexpf((float)v.w, -sh);
    *pc = make_int4(0, 0, 0, 0);
  }
}

// Issue balance between the two waves of a SIMD in an 8-wave workgroup (waves w and
// w + 4): at equal priority the older wave wins the issue slot, finishes its work long
// before the younger one and leaves it streaming alone.  Each wave counts the blocks it
// has started in `progress` (kWaves ints of workgroup memory, zeroed before the first
// call); the result is true, uniform over the wave, while this wave has started fewer
// blocks than its partner, and the caller then raises its priority one level.
template <int kWaves>
__device__ __forceinline__ bool behind_partner(int* progress, int lane) {
  static_assert(kWaves == 8, "partners w and w + 4");
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (lane == 0) __hip_atomic_fetch_add(&progress[wv], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const int mine = __hip_atomic_load(&progress[wv], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const int theirs = __hip_atomic_load(&progress[wv ^ (kWaves / 2)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(mine < theirs ? 1 : 0) != 0;
}

}  // namespace dcm
}  // namespace kvq
