// chunk_mfma.hip -- causal attention of a chunk of query tokens over the packed cache,
// on the matrix cores of gfx950: uniform 4-bit keys, 2/4-bit values, head_dim 128,
// 128-token blocks, value groups of 64 or 128, 0 to 2 sparse outliers per vector.
//
// Pages cited (title, address):
//   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
//   [UQ]   "大模型长上下文推理优化：4-bit KV Cache量化技术解析与部署实践", mlqm.cn/news/1064729
//   [TQ]   "TurboQuant：突破大模型推理瓶颈的KVCache量化技术解析", mlqm.cn/news/1002276
//
// A chunk of nq query tokens (a prefill chunk, or the draft tokens of a speculative
// verification step; [UQ] section 5.1 counts first-token latency among the costs) turns
// the decode's matrix-vector products into real contractions.  The R = (q_heads /
// kv_heads) * nq query vectors of a kv head ("rows": query head g, query j at position
// q_pos + j) form tiles of 16, and per 128-token block both products run on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//  * scores: S^T[token][row] = sum over the 128 slots (pair i, re/im) of
//    K[token][slot] W[slot][row], K the dequantized key pair (k_i, k_{i+64}) rotated by
//    the token's offset j in the block ([KVC3] "Pre-RoPE Key Quantization": RoPE after
//    dequantization), W = conj(q) e^{i f (n Bk - p)} the query weights with the block's
//    and the query's rotations folded in;
//  * values: O^T[channel][row] += sum_t code[t][channel] w[t][row], the integer codes
//    exact in fp16 and w = p * scale the value weights; the zero-points add
//    sum_t p_t zero_t per row in fp32 ([KVC3] "Quanto 的量化原理": x = s c + z).
// fp16 operands carry fp32 values as hi + lo (hi = x rounded toward zero, lo = the
// remainder rounded the same way: |x - hi - lo| <= 2^-20 |x|), and each product takes
// three MFMAs (hi hi, hi lo, lo hi; the dropped lo lo term is below 2^-20 of the
// product): the split-operand method of Markidis et al. (2018, "NVIDIA Tensor Core
// Programmability, Performance & Precision") and Ootomo & Yokota (2022).  Every operand
// is scaled by a power of two so that its largest possible magnitude lies in
// [2^14, 2^15): keys per block (from the block's scales and zero-points), queries per
// row, value weights per row and block (from the block's largest p and scale).  So no
// fp16 overflows, and fp16 subnormals (flushed or not) weigh at most 2^-28 of that
// largest magnitude.  Nothing is dequantized to memory ([TQ] sections 5.1 and 6.3).
//
// Lane l = 16 g + m of a wave.  In the score MFMA the lane supplies key row m (a token)
// with the 8 slots of pairs 16 g + 4 kappa .. + 3 (kappa = the 32-slot chunk), and
// query column m (a row) with the same slots; it receives S^T rows 4 g + v (v < 4) of
// column m, i.e. the scores of ITS row m at 4 tokens per 16-token tile.  The token of
// tile tau and output row 4 g + v is chosen so that tiles 2 kp and 2 kp + 1 give the lane
// exactly the 8 tokens of one packed value word (4-bit: tokens 32 kp + 8 g + 0..7;
// 2-bit: two 4-token runs of one 16-token word).  The value MFMA then takes the lane's
// own probabilities as its B operand (column m = row m, the same 8 tokens as k slots)
// with no exchange between lanes, and the lane's A operand is the codes of channels
// 64 h + 4 m + c (c < 4) from one 16-byte load.
//
// Sparse outliers ([KVC3] "Per-Vector Dense-and-Sparse Quantization": code 0 is stored
// at an outlier, its exact fp16 value in the CSR):
//  * keys: per (token, entry) one lane forms the rotated difference
//    D = (x - zero) e^{i f_i j} e^{i f_i n Bk} (the block rotation moved off the query);
//    every row then adds Re(Wq D) to its score, Wq read from LDS: 2 FMAs per term;
//  * values: p * (x - zero) per (row, token, entry), fixed point with one shift per
//    block (from the block's largest |x - zero|), LDS integer adds into a per-wave
//    [row][channel] array, merged into the output tiles after the block.
//
// Work: a workgroup takes kCW consecutive splits of a unit (b, kv-head, row tile), one
// per wave (split s takes blocks s, s + S, ... below the tile's last visible block), so
// its waves share the unit's query weights and stream neighbouring blocks.  The
// unquantized tail is left to the finish kernel.
#include <math.h>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dcm;

// waves per workgroup: 8 (two per SIMD, 256 registers each) without outliers; 4 (one per
// SIMD, 512 registers) with them, whose per-wave LDS (difference and correction arrays)
// and registers do not fit eight
template <int KO>
constexpr int cw_of() { return KO ? 4 : 8; }

// Blocks each wave of an 8-wave workgroup has started (waves w and w + 4 share a SIMD):
// the wave behind its partner runs at a raised priority, so that the older wave of a
// SIMD does not finish its split long before the younger one (the next unit's barrier
// would wait for it).
__shared__ int chunk_progress[8];
constexpr int kD = 128, kBK = 128, kHalf = 64;
constexpr int kTP = kD + 4;                 // floats per rotary-table row
constexpr int kRows = 16;                   // rows per tile
constexpr int kWQP = 2 * kHalf + 4;         // floats per row of the query weights
constexpr int kVCP = kD + 4;                // ints per row of the value-outlier sums (banks)

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// D += A B: lane l supplies row l % 16 of A and column l % 16 of B, 8 entries each of
// the 32-long reduction index (the same 8 positions in both), and receives
// D[4 (l / 16) + v][l % 16] in element v.
__device__ __forceinline__ f4 mfma16(u4v a, u4v b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0,
                                                0);
}

// Two fp32 values as fp16 (rounded toward zero) in one dword, and their remainders
// x - hi (exact in fp32, then rounded toward zero) in another.  `neg1` is -1.0 passed
// in from the host: as a value the compiler cannot see, x + neg1 * hi stays one mixed
// fp16/fp32 fused multiply-add (v_fma_mix_f32) instead of a conversion and a subtraction.
__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo, float neg1) {
  hi = pk_rtz(a, b);
  const h2t h = __builtin_bit_cast(h2t, hi);
  lo = pk_rtz(__builtin_fmaf((float)h.x, neg1, a), __builtin_fmaf((float)h.y, neg1, b));
}

// The exponent e with bound * 2^e in [2^14, 2^15) (bound > 0).
__device__ __forceinline__ int exp_to_2p15(float bound) { return 15 - __builtin_amdgcn_frexp_expf(bound); }

// Token offset in the block of tile tau, output row 4 g + v (see the file comment).
template <int VB>
__host__ __device__ inline int tok_of(int tau, int g, int v) {
  if constexpr (VB == 4) return 32 * (tau >> 1) + 8 * g + 4 * (tau & 1) + v;
  else return 32 * (tau >> 1) + 16 * (g >> 1) + 4 * (g & 1) + 8 * (tau & 1) + v;
}
// Inverse: the slot 16 tau + 4 g + v of token offset t.
template <int VB>
__host__ __device__ inline int slot_of(int t) {
  const int a = t >> 5, v = t & 3;
  if constexpr (VB == 4) {
    const int g = (t >> 3) & 3, b = (t >> 2) & 1;
    return 16 * (2 * a + b) + 4 * g + v;
  } else {
    const int g = 2 * ((t >> 4) & 1) + ((t >> 2) & 1), b = (t >> 3) & 1;
    return 16 * (2 * a + b) + 4 * g + v;
  }
}

// Per-wave LDS area, in floats.
struct CLds {
  int meta, eb, vs, vz, de, vcs, vc, total;
};
__host__ __device__ inline CLds chunk_lds(int ng, int ko) {
  CLds m;
  int o = 0;
  m.meta = o; o += 4 * kHalf;   // per pair: scale_a 2^(24+ek), zero_a 2^ek, scale_b 2^(20+ek), zero_b 2^ek
  m.eb = o; o += 2 * kHalf;     // per pair: cos/sin(n Bk f_i)
  m.vs = o; o += ng * kBK;      // value scales, [group][slot]
  m.vz = o; o += ng * kBK;      // value zero-points, [group][slot]
  m.vcs = o; o += ko ? 2 * kBK : 0;        // value outliers: (columns, values) per token
  // one area, used in turn: the key-outlier score terms [token][row] (block start to the
  // scores' correction), then the value-outlier sums [row][channel] in fixed point
  m.de = o;
  m.vc = o;
  o += ko ? (kBK * kRows > kRows * kVCP ? kBK * kRows : kRows * kVCP) : 0;
  m.total = o;
  return m;
}
// Workgroup LDS, in floats: rotary table, query weights, per-row exponents, wave areas.
__host__ __device__ inline int chunk_lds_total(int ng, int ko, int cw) {
  return kBK * kTP + kRows * kWQP + kRows + cw * chunk_lds(ng, ko).total;
}

template <int VB>
struct CRegs {
  static constexpr int TPW = 32 / VB;  // tokens per value word
  uint4 k[8];        // key bytes 16 g .. 16 g + 15 of the token of tile tau, row m
  uint4 v[4][2];     // value words of the lane's 8 tokens of chunk kp, channels 64 h + 4 m ..
  uint16_t kmeta[4]; // lane i: scale[i], scale[i + 64], zero[i], zero[i + 64]
  float2 eb;         // lane i: cos/sin(n Bk f_i)
  uint32_t vs[2], vz[2];  // value scale/zero of tokens lane, 64 + lane (both groups)
  uint32_t kc[2], kv[2], vc[2], vv[2];  // outliers of tokens lane, 64 + lane: columns (byte e), values (half e)
};

// Buffer resources of one (b, kv-head): the head's slice of each buffer, with its exact
// size as the record count (a load outside it returns 0 instead of touching other
// memory).  Loads then take a lane-constant 32-bit offset and a wave-uniform block
// offset, so block addresses cost no vector registers.
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 family: raw (untyped) buffer access
struct CRsrc {
  __amdgpu_buffer_rsrc_t k, v, ks, kz, vs, vz, rope, kcol, kval, vcol, vval;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kRsrcWord3);
}
template <int VB, int NG, int KO>
__device__ __forceinline__ CRsrc head_rsrc(const kvq_cache& c, int64_t bh) {
  const int64_t T = c.cfg.capacity;
  CRsrc r;
  r.k = rsrc(static_cast<const uint8_t*>(c.k_codes) + bh * T * (kD / 2), T * (kD / 2));
  r.v = rsrc(static_cast<const uint8_t*>(c.v_codes) + bh * T * (kD * VB / 8), T * (kD * VB / 8));
  r.ks = rsrc(c.k_scale + bh * (T / kBK) * kD, (T / kBK) * kD * 2);
  r.kz = rsrc(c.k_zero + bh * (T / kBK) * kD, (T / kBK) * kD * 2);
  r.vs = rsrc(c.v_scale + bh * T * NG, T * NG * 2);
  r.vz = rsrc(c.v_zero + bh * T * NG, T * NG * 2);
  r.rope = rsrc(c.rope, ((int64_t)kBK + T / kBK) * kD * 4);
  if constexpr (KO > 0) {
    r.kcol = rsrc(c.k_col + bh * T * KO, T * KO);
    r.kval = rsrc(c.k_val + bh * T * KO, T * KO * 2);
    r.vcol = rsrc(c.v_col + bh * T * KO, T * KO);
    r.vval = rsrc(c.v_val + bh * T * KO, T * KO * 2);
  }
  return r;
}

template <int VB>
__device__ __forceinline__ void cload_k(CRegs<VB>& R, int tau, const CRsrc& rs, int64_t n, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const int t = tok_of<VB>(tau, m >> 2, m & 3);
  R.k[tau] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs.k, t * (kD / 2) + 16 * g, (int)(n * kBK * (kD / 2)), 0));
}
template <int VB>
__device__ __forceinline__ void cload_v(CRegs<VB>& R, int kp, int h, const CRsrc& rs, int64_t n, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const int word = VB == 4 ? 4 * kp + g : 2 * kp + (g >> 1);
  R.v[kp][h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs.v, (word * kD + 64 * h + 4 * m) * 4, (int)(n * kBK * kD * VB / 8), 0));
}
template <int VB, int NG, int KO>
__device__ __forceinline__ void cload_meta(CRegs<VB>& R, const CRsrc& rs, int64_t n, int lane) {
  const int kb = (int)(n * kD * 2);
  R.kmeta[0] = __builtin_amdgcn_raw_buffer_load_b16(rs.ks, 2 * lane, kb, 0);
  R.kmeta[1] = __builtin_amdgcn_raw_buffer_load_b16(rs.ks, 2 * (lane + kHalf), kb, 0);
  R.kmeta[2] = __builtin_amdgcn_raw_buffer_load_b16(rs.kz, 2 * lane, kb, 0);
  R.kmeta[3] = __builtin_amdgcn_raw_buffer_load_b16(rs.kz, 2 * (lane + kHalf), kb, 0);
  R.eb = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rs.rope, 8 * lane,
                                                                          (int)(((int64_t)kBK + n) * kD * 4), 0));
  const int vb = (int)(n * kBK * NG * 2);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int t = kWave * k + lane;
    if constexpr (NG == 2) {
      R.vs[k] = __builtin_amdgcn_raw_buffer_load_b32(rs.vs, 4 * t, vb, 0);
      R.vz[k] = __builtin_amdgcn_raw_buffer_load_b32(rs.vz, 4 * t, vb, 0);
    } else {
      R.vs[k] = __builtin_amdgcn_raw_buffer_load_b16(rs.vs, 2 * t, vb, 0);
      R.vz[k] = __builtin_amdgcn_raw_buffer_load_b16(rs.vz, 2 * t, vb, 0);
    }
  }
  if constexpr (KO > 0) {
    const int cb = (int)(n * kBK * KO);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = kWave * k + lane;
      if constexpr (KO == 2) {
        R.kc[k] = __builtin_amdgcn_raw_buffer_load_b16(rs.kcol, 2 * t, cb, 0);
        R.vc[k] = __builtin_amdgcn_raw_buffer_load_b16(rs.vcol, 2 * t, cb, 0);
        R.kv[k] = __builtin_amdgcn_raw_buffer_load_b32(rs.kval, 4 * t, 2 * cb, 0);
        R.vv[k] = __builtin_amdgcn_raw_buffer_load_b32(rs.vval, 4 * t, 2 * cb, 0);
      } else {
        R.kc[k] = __builtin_amdgcn_raw_buffer_load_b8(rs.kcol, t, cb, 0);
        R.vc[k] = __builtin_amdgcn_raw_buffer_load_b8(rs.vcol, t, cb, 0);
        R.kv[k] = __builtin_amdgcn_raw_buffer_load_b16(rs.kval, 2 * t, 2 * cb, 0);
        R.vv[k] = __builtin_amdgcn_raw_buffer_load_b16(rs.vval, 2 * t, 2 * cb, 0);
      }
    }
  }
}

// Running state of the lane's row m over one split.
struct CState {
  float m;        // running max (base 2)
  float l;        // partial sum of p over the lane's tokens
  float z[2];     // partial sum of p * zero over the lane's tokens, per group
  int e;          // o is held at scale 2^(e - 18) (4-bit) or 2^(e - 16) (2-bit): weights at 2^e
  f4 o[8];        // O^T tiles 4 h + c: element v = channel 64 h + 16 g + 4 v + c of row m
};

template <int VB, int NG, int KO>
__device__ __forceinline__ void chunk_block(CRegs<VB>& R, const CRsrc& rs, CState& st, float* __restrict__ wl,
                                            const CLds& L,
                                            const float* __restrict__ table, const float* __restrict__ wq,
                                            int eq, int lane, const kvq_cache& c, int64_t bh, int64_t n,
                                            int64_t nn, bool more, int64_t vis_row, bool masked, float neg1) {
  const int m = lane & 15, g = lane >> 4;
  float* Meta = wl + L.meta;
  float* EB = wl + L.eb;
  float* VS = wl + L.vs;
  float* VZ = wl + L.vz;

  // ---- block constants into LDS: key scale/zero at 2^ek (the block's largest rotated
  // key below 2^15), the block rotation, the value metadata in slot order
  int ek;
  float vsmax;
  {
    const float sa = h2f(R.kmeta[0]), sb = h2f(R.kmeta[1]), za = h2f(R.kmeta[2]), zb = h2f(R.kmeta[3]);
    // |k| <= max(|z|, |z + 15 s|) (codes 0..15); a rotated pair is at most sqrt(2) max |k|
    const float ka = fmaxf(fabsf(za), fabsf(fmaf(15.0f, sa, za)));
    const float kb = fmaxf(fabsf(zb), fabsf(fmaf(15.0f, sb, zb)));
    const float kmax = wave_max_uniform(fmaxf(ka, kb)) * 1.4142137f;
    ek = kmax > 0.0f ? exp_to_2p15(kmax) : 0;
    *reinterpret_cast<float4*>(Meta + 4 * lane) =
        make_float4(__builtin_amdgcn_ldexpf(sa, 24 + ek), __builtin_amdgcn_ldexpf(za, ek),
                    __builtin_amdgcn_ldexpf(sb, 20 + ek), __builtin_amdgcn_ldexpf(zb, ek));
    *reinterpret_cast<float2*>(EB + 2 * lane) = R.eb;
    float vmx = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int sl = slot_of<VB>(kWave * k + lane);
#pragma unroll
      for (int grp = 0; grp < NG; ++grp) {
        const float s = h2f((uint16_t)(R.vs[k] >> (16 * grp)));
        VS[grp * kBK + sl] = s;
        VZ[grp * kBK + sl] = h2f((uint16_t)(R.vz[k] >> (16 * grp)));
        vmx = fmaxf(vmx, s);
      }
    }
    vsmax = wave_max_uniform(vmx);
  }
  // value outliers of the lane's two tokens: staged per token for the lanes that hold
  // their probabilities, and the block's largest |x - zero| for the fixed-point shift
  int shv = 0;
  if constexpr (KO > 0) {
    uint32_t* VCS = reinterpret_cast<uint32_t*>(wl + L.vcs);
    float dmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = kWave * k + lane;
      *reinterpret_cast<uint2*>(VCS + 2 * t) = make_uint2(R.vc[k], R.vv[k]);
#pragma unroll
      for (int e = 0; e < KO; ++e) {
        const int col = (int)((R.vc[k] >> (8 * e)) & 0xffu);
        const int grp = NG == 2 ? col >> 6 : 0;
        const float z = h2f((uint16_t)(R.vz[k] >> (16 * grp)));
        dmax = fmaxf(dmax, fabsf(h2f((uint16_t)(R.vv[k] >> (16 * e))) - z));
      }
    }
    // a channel sums at most 128 terms |p (x - z)| <= dmax < 2^ed: each term below 2^23
    // after the shift, every channel sum below 2^30
    shv = 23 - __builtin_amdgcn_frexp_expf(wave_max_uniform(dmax));
  }
  const uint32_t kcn[2] = {R.kc[0], R.kc[1]}, kvn[2] = {R.kv[0], R.kv[1]};  // this block's key outliers
  if (more) cload_meta<VB, NG, KO>(R, rs, nn, lane);
  wave_lds_sync();

  // ---- key outliers: per (token, entry) the rotated difference D = (x - zero) e^{i f_i
  // (n Bk + j)} in the keys' scale 2^ek, and its score term Re(Wq D) for all 16 rows,
  // summed over the token's entries into the [token][row] array (lane: tokens lane and
  // 64 + lane); the rows add them after the score MFMAs
  if constexpr (KO > 0) {
    float* DE = wl + L.de;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = kWave * k + lane;
      float dx[KO], dy[KO];
      int ie[KO];
#pragma unroll
      for (int e = 0; e < KO; ++e) {
        const int col = (int)((kcn[k] >> (8 * e)) & 0xffu);
        const int i = col & (kHalf - 1);
        const bool isb = col >= kHalf;
        const float4 M = *reinterpret_cast<const float4*>(Meta + 4 * i);
        const float d = __builtin_amdgcn_ldexpf(h2f((uint16_t)(kvn[k] >> (16 * e))), ek) - (isb ? M.w : M.y);
        const float2 cssn = *reinterpret_cast<const float2*>(table + t * kTP + ((2 * i) ^ (t & 16)));
        const float2 eb = *reinterpret_cast<const float2*>(EB + 2 * i);
        const float x = isb ? -d * cssn.y : d * cssn.x, y = isb ? d * cssn.x : d * cssn.y;
        dx[e] = eb.x * x - eb.y * y;
        dy[e] = eb.y * x + eb.x * y;
        ie[e] = i;
      }
#pragma unroll
      for (int r4 = 0; r4 < kRows / 4; ++r4) {
        float cr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          cr[u] = 0.0f;
#pragma unroll
          for (int e = 0; e < KO; ++e) {
            const float2 w = *reinterpret_cast<const float2*>(wq + (4 * r4 + u) * kWQP + 2 * ie[e]);
            cr[u] = __builtin_fmaf(w.x, dx[e], __builtin_fmaf(-w.y, dy[e], cr[u]));
          }
        }
        *reinterpret_cast<float4*>(DE + t * kRows + 4 * r4) = make_float4(cr[0], cr[1], cr[2], cr[3]);
      }
    }
    wave_lds_sync();
  }

  // ---- scores: S[tau] = S^T rows 4 g + v of tile tau, column m (the lane's row)
  f4 S[8];
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) S[tau] = f4{0.f, 0.f, 0.f, 0.f};
  // rotary table row of the lane's token, 16-float chunks swapped on rows 16..31 mod 32
  // (tsw): the 16 tokens a wave reads at once then hit 16 different 4-bank groups
  const int tsw = ((m >> 3) & 1) << 4;
  float4 t01, t23;
  {
    const float* tr = table + tok_of<VB>(0, m >> 2, m & 3) * kTP;
    t01 = *reinterpret_cast<const float4*>(tr + ((32 * g) ^ tsw));
    t23 = *reinterpret_cast<const float4*>(tr + ((32 * g + 4) ^ tsw));
  }
#pragma unroll
  for (int kap = 0; kap < 4; ++kap) {
    const int p0 = 16 * g + 4 * kap;  // the chunk's first pair for this lane
    // query operand: slots (W_r, -W_i) of pairs p0 .. p0 + 3 of row m, W = Wq e^{i n Bk f}
    u4v Bh, Bl;
    {
      const float4 w01 = *reinterpret_cast<const float4*>(wq + m * kWQP + 2 * p0);
      const float4 w23 = *reinterpret_cast<const float4*>(wq + m * kWQP + 2 * p0 + 4);
      const float4 e01 = *reinterpret_cast<const float4*>(EB + 2 * p0);
      const float4 e23 = *reinterpret_cast<const float4*>(EB + 2 * p0 + 4);
      const float qr[4] = {w01.x, w01.z, w23.x, w23.z}, qi[4] = {w01.y, w01.w, w23.y, w23.w};
      const float ec[4] = {e01.x, e01.z, e23.x, e23.z}, es[4] = {e01.y, e01.w, e23.y, e23.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wr = qr[u] * ec[u] - qi[u] * es[u];
        const float wi = qr[u] * es[u] + qi[u] * ec[u];
        uint32_t hi, lo;
        split2(wr, -wi, hi, lo, neg1);
        Bh[u] = hi;
        Bl[u] = lo;
      }
    }
    float4 M[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) M[u] = *reinterpret_cast<const float4*>(Meta + 4 * (p0 + u));
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      // the next iteration's cos/sin, read ahead of this one's arithmetic
      float4 tn01 = t01, tn23 = t23;
      if (tau < 7 || kap < 3) {
        const int tn = tau < 7 ? tau + 1 : 0, pn = tau < 7 ? p0 : p0 + 4;
        const float* tr = table + tok_of<VB>(tn, m >> 2, m & 3) * kTP;
        tn01 = *reinterpret_cast<const float4*>(tr + ((2 * pn) ^ tsw));
        tn23 = *reinterpret_cast<const float4*>(tr + ((2 * pn + 4) ^ tsw));
      }
      const uint32_t x = kap == 0 ? R.k[tau].x : kap == 1 ? R.k[tau].y : kap == 2 ? R.k[tau].z : R.k[tau].w;
      // nibbles masked into bits 0-3 / 4-7 of a 16-bit half are exact fp16 subnormals
      // (code * 2^-24, code * 2^-20), read in place by the dequantizing FMAs
      const uint32_t t8 = x >> 8;
      const h2t a02 = __builtin_bit_cast(h2t, x & 0x000F000Fu), b02 = __builtin_bit_cast(h2t, x & 0x00F000F0u);
      const h2t a13 = __builtin_bit_cast(h2t, t8 & 0x000F000Fu), b13 = __builtin_bit_cast(h2t, t8 & 0x00F000F0u);
      const float ca[4] = {(float)a02.x, (float)a13.x, (float)a02.y, (float)a13.y};
      const float cb[4] = {(float)b02.x, (float)b13.x, (float)b02.y, (float)b13.y};
      const float cs[4] = {t01.x, t01.z, t23.x, t23.z}, sn[4] = {t01.y, t01.w, t23.y, t23.w};
      u4v Ah, Al;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float ka = __builtin_fmaf(M[u].x, ca[u], M[u].y);
        const float kb = __builtin_fmaf(M[u].z, cb[u], M[u].w);
        const float X = __builtin_fmaf(ka, cs[u], -(kb * sn[u]));
        const float Y = __builtin_fmaf(ka, sn[u], kb * cs[u]);
        uint32_t hi, lo;
        split2(X, Y, hi, lo, neg1);
        Ah[u] = hi;
        Al[u] = lo;
      }
      S[tau] = mfma16(Ah, Bh, S[tau]);
      S[tau] = mfma16(Ah, Bl, S[tau]);
      S[tau] = mfma16(Al, Bh, S[tau]);
      if (kap == 3 && more) cload_k<VB>(R, tau, rs, nn, lane);
      t01 = tn01;
      t23 = tn23;
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if constexpr (KO > 0) {  // key-outlier terms of the lane's row; the area then holds the value sums
    float* DE = wl + L.de;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
#pragma unroll
      for (int v = 0; v < 4; ++v) S[tau][v] += DE[tok_of<VB>(tau, g, v) * kRows + m];
    wave_lds_sync();
    for (int k = 4 * lane; k < kRows * kVCP; k += 4 * kWave)
      *reinterpret_cast<int4*>(DE + k) = make_int4(0, 0, 0, 0);
  }

  // ---- online softmax of row m (base 2; the query weights carry log2(e) / sqrt(D))
  const float unscale = __builtin_amdgcn_ldexpf(1.0f, -(ek + eq));
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) S[tau] *= unscale;
  if (masked) {  // the block reaches past the view of some row: hide the tokens it does not see
    const int64_t seen64 = vis_row - n * kBK;
    const int seen = seen64 < 0 ? 0 : (seen64 > kBK ? kBK : (int)seen64);
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (tok_of<VB>(tau, g, v) >= seen) S[tau][v] = -__builtin_inff();
  }
  float mloc = -__builtin_inff();
#pragma unroll
  for (int tau = 0; tau < 8; ++tau)
#pragma unroll
    for (int v = 0; v < 4; ++v) mloc = fmaxf(mloc, S[tau][v]);
  // the row's 128 tokens sit in lanes m, m + 16, m + 32, m + 48
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
  const float mnew = fmaxf(st.m, mloc);
  const float msafe = mnew == -__builtin_inff() ? 0.0f : mnew;  // a row that has seen nothing yet
  const float alpha = __builtin_amdgcn_exp2f(st.m - msafe);
  const float pmax = __builtin_amdgcn_exp2f(mloc - msafe);
  st.m = mnew;
  float lsum = 0.0f;
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      S[tau][v] = __builtin_amdgcn_exp2f(S[tau][v] - msafe);
      lsum += S[tau][v];
    }
  }
  st.l = __builtin_fmaf(st.l, alpha, lsum);
  // value weights p * scale at 2^E: the block's largest weight of this row in [2^14, 2^15).
  // pmax counts as at least 2^-24: a block whose weights all lie below 2^-24 of the
  // running maximum's adds nothing the accumulator can hold, and the cap keeps E from
  // growing so fast that the rescaled accumulator (o * 2^(E - E_old)) overflows
  const float wbound = fmaxf(pmax, 0x1p-24f) * vsmax;
  const int E = wbound > 0.0f ? exp_to_2p15(wbound) : st.e;
  const float ao = __builtin_amdgcn_ldexpf(alpha, E - st.e);
  st.e = E;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.o[t] *= ao;

  // ---- value outliers: p (x - zero) into the [row][channel] array (fixed point at 2^shv)
  if constexpr (KO > 0) {
    const uint32_t* VCS = reinterpret_cast<const uint32_t*>(wl + L.vcs);
    int* VC = reinterpret_cast<int*>(wl + L.vc);
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = tok_of<VB>(tau, g, v);
        const uint2 cv = *reinterpret_cast<const uint2*>(VCS + 2 * t);
        const float ps = __builtin_amdgcn_ldexpf(S[tau][v], shv);
#pragma unroll
        for (int e = 0; e < KO; ++e) {
          const int col = (int)((cv.x >> (8 * e)) & 0xffu);
          const int grp = NG == 2 ? col >> 6 : 0;
          const float z = VZ[grp * kBK + 16 * tau + 4 * g + v];
          const float term = ps * (h2f((uint16_t)(cv.y >> (16 * e))) - z);
          atomicAdd(VC + m * kVCP + col, (int)__builtin_rintf(term));
        }
      }
  }

  // ---- values: O^T[channel][row] += codes x weights, per 32-token chunk kp
#pragma unroll
  for (int kp = 0; kp < 4; ++kp) {
    u4v Wh[NG], Wl[NG];
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      const float4 sa = *reinterpret_cast<const float4*>(VS + grp * kBK + 16 * (2 * kp) + 4 * g);
      const float4 sb = *reinterpret_cast<const float4*>(VS + grp * kBK + 16 * (2 * kp + 1) + 4 * g);
      const float4 za = *reinterpret_cast<const float4*>(VZ + grp * kBK + 16 * (2 * kp) + 4 * g);
      const float4 zb = *reinterpret_cast<const float4*>(VZ + grp * kBK + 16 * (2 * kp + 1) + 4 * g);
      const float s0[4] = {sa.x, sa.y, sa.z, sa.w}, s1[4] = {sb.x, sb.y, sb.z, sb.w};
      const float z0[4] = {za.x, za.y, za.z, za.w}, z1[4] = {zb.x, zb.y, zb.z, zb.w};
      float zs = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p0 = S[2 * kp][v], p1 = S[2 * kp + 1][v];
        zs = __builtin_fmaf(p0, z0[v], __builtin_fmaf(p1, z1[v], zs));
        uint32_t hi, lo;
        split2(__builtin_amdgcn_ldexpf(p0 * s0[v], E), __builtin_amdgcn_ldexpf(p1 * s1[v], E), hi, lo, neg1);
        Wh[grp][v] = hi;
        Wl[grp][v] = lo;
      }
      st.z[grp] = kp == 0 ? __builtin_fmaf(st.z[grp], alpha, zs) : st.z[grp] + zs;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int grp = NG == 2 ? h : 0;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const uint32_t w = cc == 0 ? R.v[kp][h].x : cc == 1 ? R.v[kp][h].y : cc == 2 ? R.v[kp][h].z : R.v[kp][h].w;
        // dword k holds the codes of the tokens of output elements (tile 2 kp, v = k) and
        // (tile 2 kp + 1, v = k), moved into the top bits of the two halves' mantissas:
        // exact fp16 subnormals code * 2^-18 (4-bit, bits 6-9) or code * 2^-16 (2-bit,
        // bits 8-9).  The matrix cores keep fp16 subnormal inputs, but sum products at the
        // precision of the smallest normal exponent: codes in the low mantissa bits would
        // lose up to 9 bits there, at the top at most 3.
        u4v A;
        if constexpr (VB == 4) {
          A[0] = (w << 6) & 0x03C003C0u;  // nibbles 0, 4
          A[1] = (w << 2) & 0x03C003C0u;  // nibbles 1, 5
          A[2] = (w >> 2) & 0x03C003C0u;  // nibbles 2, 6
          A[3] = (w >> 6) & 0x03C003C0u;  // nibbles 3, 7
        } else {
          const uint32_t ws = w >> (8 * (g & 1));
#pragma unroll
          for (int k = 0; k < 4; ++k) A[k] = (ws << (8 - 2 * k)) & 0x03000300u;  // fields k, k + 8
        }
        st.o[4 * h + cc] = mfma16(A, Wh[grp], st.o[4 * h + cc]);
        st.o[4 * h + cc] = mfma16(A, Wl[grp], st.o[4 * h + cc]);
      }
      if (more) cload_v<VB>(R, kp, h, rs, nn, lane);
    }
  }
  if (NG == 1) st.z[1] = 0.0f;
  if constexpr (KO > 0) {  // this block's value-outlier sums into the output tiles
    wave_lds_sync();
    constexpr int kCodeExp = VB == 4 ? 18 : 16;
    int* VC = reinterpret_cast<int*>(wl + L.vc);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int4* pc = reinterpret_cast<int4*>(VC + m * kVCP + 64 * h + 16 * g + 4 * v);
        const int4 x = *pc;
        const int sc = E - kCodeExp - shv;
        st.o[4 * h][v] += __builtin_amdgcn_ldexpf((float)x.x, sc);
        st.o[4 * h + 1][v] += __builtin_amdgcn_ldexpf((float)x.y, sc);
        st.o[4 * h + 2][v] += __builtin_amdgcn_ldexpf((float)x.z, sc);
        st.o[4 * h + 3][v] += __builtin_amdgcn_ldexpf((float)x.w, sc);
      }
  }
  wave_lds_sync();
}

template <int VB, int NG, int KO>
__global__ __launch_bounds__(cw_of<KO>() * 64) void chunk_mfma_kernel(kvq_cache c, const uint16_t* __restrict__ q,
                                                              RowSpec rs, float* __restrict__ ws, int S,
                                                              int ntiles, int64_t nwork, float neg1) {
  constexpr int kCW = cw_of<KO>();
  constexpr int kNT = kCW * 64;
  extern __shared__ float lds[];
  const int H = c.cfg.kv_heads, Hq = c.cfg.q_heads, gq = Hq / H, R = gq * rs.nq;
  const int64_t nfull = c.length / kBK;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;

  float* table = lds;
  float* wq = lds + kBK * kTP;  // [row][pair] (re, im) at 2^eq_row
  int* eqs = reinterpret_cast<int*>(wq + kRows * kWQP);
  const CLds L = chunk_lds(NG, KO);
  float* wl = lds + kBK * kTP + kRows * kWQP + kRows + wave * L.total;
  for (int idx = threadIdx.x; idx < kBK * kHalf; idx += kNT) {
    const int j = idx / kHalf, i = idx % kHalf;
    *reinterpret_cast<float2*>(table + j * kTP + ((2 * i) ^ (j & 16))) = *reinterpret_cast<const float2*>(c.rope + 2 * idx);
  }

  const int nsg = (S + kCW - 1) / kCW;  // split groups per unit
  if (threadIdx.x < 8) chunk_progress[threadIdx.x] = 0;  // published by the loop's first barrier
  for (int64_t work = blockIdx.x; work < nwork; work += gridDim.x) {
    const int sg = (int)(work % nsg);
    const int64_t unit = work / nsg;
    const int tile = (int)(unit % ntiles);
    const int64_t bh = unit / ntiles;
    const int h = (int)(bh % H);
    const int b = (int)(bh / H);
    __syncthreads();  // the previous unit is done with the query weights
    // ---- query weights of the tile: wave w computes rows w, w + kCW, ... (lane = pair):
    // scale * conj(q) e^{-i f p} in fp64, then the row at 2^eq (its largest weight's
    // magnitude below 2^15)
    for (int r = wave; r < kRows; r += kCW) {
      const int row = tile * kRows + r;
      float wr = 0.0f, wi = 0.0f;
      if (row < R) {
        const int qj = row % rs.nq;
        const uint16_t* qv = q + (((int64_t)b * Hq + (int64_t)h * gq + row / rs.nq) * rs.nq + qj) * kD;
        const double f = pow((double)c.cfg.rope_theta, -(2.0 * lane) / (double)kD);
        double sn, cs;
        sincos((double)(rs.q_pos + qj) * f, &sn, &cs);
        const double scl = (double)kLog2e / sqrt((double)kD);
        const double qa = (double)h2f(qv[lane]), qb = (double)h2f(qv[lane + kHalf]);
        wr = (float)(scl * (qa * cs - qb * sn));
        wi = (float)(-scl * (qa * sn + qb * cs));
      }
      const float wmax = wave_max_uniform(fabsf(wr) + fabsf(wi));
      const int eq = wmax > 0.0f ? exp_to_2p15(wmax) : 0;
      *reinterpret_cast<float2*>(wq + r * kWQP + 2 * lane) =
          make_float2(__builtin_amdgcn_ldexpf(wr, eq), __builtin_amdgcn_ldexpf(wi, eq));
      if (lane == 0) eqs[r] = eq;
    }
    __syncthreads();

    // rows of the tile: the lane's row m, and the tile's narrowest and widest views
    const int myrow = tile * kRows + m;
    const int64_t vis_row = myrow < R ? row_visible(rs, myrow % rs.nq, c.length) : c.length;
    int64_t vmin = c.length, vmax = 0;
    for (int r = 0; r < kRows && tile * kRows + r < R; ++r) {
      const int64_t v = row_visible(rs, (tile * kRows + r) % rs.nq, c.length);
      vmin = v < vmin ? v : vmin;
      vmax = v > vmax ? v : vmax;
    }
    int64_t nlimit = (vmax + kBK - 1) / kBK;
    if (nlimit > nfull) nlimit = nfull;
    const int eq = eqs[m];

    const int sp = sg * kCW + wave;
    if (sp < S) {
      CState st;
      st.m = -__builtin_inff();
      st.l = 0.0f;
      st.z[0] = st.z[1] = 0.0f;
      st.e = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) st.o[t] = f4{0.f, 0.f, 0.f, 0.f};
      CRegs<VB> Rg;
      const CRsrc rsr = head_rsrc<VB, NG, KO>(c, bh);
      if (sp < nlimit) {
        cload_meta<VB, NG, KO>(Rg, rsr, sp, lane);
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) cload_k<VB>(Rg, tau, rsr, sp, lane);
#pragma unroll
        for (int kp = 0; kp < 4; ++kp)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) cload_v<VB>(Rg, kp, hh, rsr, sp, lane);
      }
      for (int64_t n = sp; n < nlimit; n += S) {
        if constexpr (kCW == 8) {
          if (behind_partner<kCW>(chunk_progress, lane)) __builtin_amdgcn_s_setprio(1);
          else __builtin_amdgcn_s_setprio(0);
        }
        const bool more = n + S < nlimit;
        const bool masked = (n + 1) * kBK > vmin;
        chunk_block<VB, NG, KO>(Rg, rsr, st, wl, L, table, wq, eq, lane, c, bh, n, more ? n + S : n, more, vis_row,
                                masked, neg1);
      }
      // ---- partial of each row: (m, l, o + z) with l, z summed over the row's 4 lanes
      float l = st.l;
      l += __shfl_xor(l, 16, kWave);
      l += __shfl_xor(l, 32, kWave);
      float z[2];
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        z[grp] = st.z[grp];
        z[grp] += __shfl_xor(z[grp], 16, kWave);
        z[grp] += __shfl_xor(z[grp], 32, kWave);
      }
      if (myrow < R) {
        float* dst = ws + ((((int64_t)b * Hq + (int64_t)h * gq + myrow / rs.nq) * rs.nq + myrow % rs.nq) * S + sp) *
                              (kD + 2);
        if (g == 0) {
          dst[0] = st.m;
          dst[1] = l;
        }
        constexpr int kCodeExp = VB == 4 ? 18 : 16;  // codes enter the value products at 2^-kCodeExp
        const float us = __builtin_amdgcn_ldexpf(1.0f, kCodeExp - st.e);  // o is at 2^(e - kCodeExp)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float zz = NG == 2 ? z[hh] : z[0];
#pragma unroll
          for (int v = 0; v < 4; ++v)
            *reinterpret_cast<float4*>(dst + 2 + 64 * hh + 16 * g + 4 * v) =
                make_float4(__builtin_fmaf(st.o[4 * hh][v], us, zz), __builtin_fmaf(st.o[4 * hh + 1][v], us, zz),
                            __builtin_fmaf(st.o[4 * hh + 2][v], us, zz), __builtin_fmaf(st.o[4 * hh + 3][v], us, zz));
        }
      }
    }
  }
}

template <int VB, int NG, int KO>
hipError_t launch_typed(const kvq_cache& c, const uint16_t* q, RowSpec rs, float* ws, int S, hipStream_t s,
                        int cus) {
  constexpr int kCW = cw_of<KO>();
  const size_t bytes = (size_t)chunk_lds_total(NG, KO, kCW) * sizeof(float);
  if (bytes + 8 * sizeof(int) > 160 * 1024) return hipErrorNotSupported;  // with the static progress counts
  hipError_t e = hipFuncSetAttribute((const void*)chunk_mfma_kernel<VB, NG, KO>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  const int R = c.cfg.q_heads / c.cfg.kv_heads * rs.nq;
  const int ntiles = (R + kRows - 1) / kRows;
  const int64_t nwork = (int64_t)c.cfg.batch * c.cfg.kv_heads * ntiles * ((S + kCW - 1) / kCW);
  const int64_t grid = nwork < cus ? nwork : cus;
  hipLaunchKernelGGL((chunk_mfma_kernel<VB, NG, KO>), dim3((unsigned)grid), dim3(kCW * 64), bytes, s, c, q, rs, ws, S,
                     ntiles, nwork, -1.0f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_mfma(const kvq_cache& c, const uint16_t* q, RowSpec rs, float* ws, int S, hipStream_t s,
                             int cus) {
  const kvq_config& g = c.cfg;
  const int ng = g.head_dim / g.v_group, ko = host_kout(g);
  // (at head_dim 128 a whole-percent outlier share gives 0 or at least 2 per vector)
  if (ko > 2 || g.k_mode != 0 || g.k_bits != 4 || g.head_dim != kD || g.k_block != kBK || g.keep_pct > 0 || g.v_mode != 0 ||
      (g.v_bits != 4 && g.v_bits != 2) || ng < 1 || ng > 2)
    return hipErrorNotSupported;
#define KVQ_CHUNK_NG(vb, ko)                                                                  \
  return ng == 2 ? launch_typed<vb, 2, ko>(c, q, rs, ws, S, s, cus)                         \
                 : launch_typed<vb, 1, ko>(c, q, rs, ws, S, s, cus);
#define KVQ_CHUNK(vb)                                                                         \
  if (g.v_bits == vb) {                                                                       \
    if (ko == 2) { KVQ_CHUNK_NG(vb, 2) }                                                      \
    if (ko == 0) { KVQ_CHUNK_NG(vb, 0) }                                                      \
  }
  KVQ_CHUNK(4) KVQ_CHUNK(2)
#undef KVQ_CHUNK
#undef KVQ_CHUNK_NG
  return hipErrorNotSupported;
}

}  // namespace kvq
