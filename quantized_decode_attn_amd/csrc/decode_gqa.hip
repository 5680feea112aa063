// decode_gqa.hip -- decode attention over uniform 4-bit keys and 2/4-bit values when
// several query heads share one kv head (grouped-query attention), tuned for gfx950.
//
// Pages cited (title, address):
//   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
//   [TQ]   "TurboQuant：突破大模型推理瓶颈的KVCache量化技术解析", mlqm.cn/news/1002276
//
// The score of query head g for token n*Bk+j is Re(sum_i W_g,i * khat_ij), where
// khat_ij = (k_a + i k_b) e^{i f_i j} is the dequantized pre-RoPE key pair ([KVC3]
// "Per-Channel Key Quantization", "Pre-RoPE Key Quantization") rotated by the token's
// offset in the block, and W_g,i = conj(q_g,i) e^{i f_i (n Bk - p)} carries the query
// rotation.  Up to four query heads of a kv head form one wave's item, and both
// contractions run on the matrix cores as fp32 v_mfma_f32_4x4x1_16b_f32, whose 16
// blocks of 4 x 4 outer products fit four heads without padding:
//  * scores: every lane owns one key token (two 64-token halves per block) and
//    computes khat for its token, pair by pair (6 VALU operations per pair: two
//    dequantizing FMAs, the rotation); per key channel one MFMA multiplies the four
//    heads' weights (lane l supplies head l % 4) with the 64 tokens' khat, so after
//    the 128 channels lane l holds the scores of its token for all four heads --
//    no cross-lane reduction;
//  * values: the weights p * scale of a block are quantized per head to 30-bit fixed
//    point (relative to a bound on the block's largest weight) and written as four
//    signed base-256 digits, so that sum_t w_t c_t is an exact integer product: one
//    v_mfma_i32_16x16x64_i8 takes the 16 rows (head, digit) against 16 channels and
//    64 tokens, the codes spread from the packed words into bytes (16 instructions
//    per block instead of 256 fp32 outer products);
//  * outliers ([KVC3] "Per-Vector Dense-and-Sparse Quantization"): code 0 was stored
//    at an outlier's position; the lane owning a token adds the exact score terms of
//    its CSR entries for every head, and scatters p * (x - zero) into a per-head
//    channel array with LDS atomics, merged at the next block's softmax.
// Blocks stream through registers as in the one-head kernel: every register slot is
// refilled with block n + 1 right after its last use in block n.  No dequantized key
// or value is written to memory ([TQ] sections 5.1 and 6.3).
#include <math.h>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dcm;

constexpr int kGqaWaves = 8;

// Blocks each wave of the workgroup has started (waves w and w + 4 share a SIMD).  As in
// the one-head kernel, the wave that has started fewer blocks than its SIMD partner runs
// one priority level higher, which keeps the older wave from finishing first and
// leaving the younger one alone on the SIMD.
__shared__ int gqa_progress[kGqaWaves];
constexpr int kD = 128, kBK = 128, kHalf = 64;
constexpr int kTP = kD + 4;  // floats per rotary-table row: 64 (cos, sin) pairs + 4 (banks)
constexpr int kWAP = 2 * kHalf + 4;  // floats per head of the query weights (distinct banks per head)
constexpr int kW32P = kHalf + 4;     // dwords per (head, token half) of the fixed-point value weights

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

typedef int i4 __attribute__((ext_vector_type(4)));
// D += A B over 64 int8 products: lane l supplies row l % 16 of A and column l % 16 of
// B, each with 16 entries of the reduction index (the same 16 positions in both), and
// receives D[4 (l / 16) + r][l % 16] in element r.
__device__ __forceinline__ i4 mfma_i8(i4 a, i4 b, i4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Per-wave LDS area, in floats.
struct GLds {
  int meta, wa, w32, vcorr, wq, total;
};
__host__ __device__ inline GLds gqa_lds(int ng, bool outl) {
  GLds m;
  int o = 0;
  m.meta = o; o += 4 * kHalf;        // per pair: scale_a / u, zero_a, scale_b / u, zero_b
  m.wa = o; o += 4 * kWAP;           // per head and pair: (W_r, -W_i)
  m.w32 = o; o += ng * 8 * kW32P;    // value weights as digits [group][head][half][lane]: token 64 half + lane
  m.vcorr = o; o += outl ? 4 * kD + 4 : 0;  // value outlier corrections [head][channel] (int), scale per head
  m.wq = o; o += kHalf * 8;          // the item's query weights per pair: (re, im) of 4 heads
  m.total = o;
  return m;
}

template <int VB>
struct GRegs {
  static constexpr int TPW = 32 / VB;   // tokens per value word
  static constexpr int WPL = 16 / TPW;  // words of one channel per 16 tokens
  static constexpr int NVI = 4 * WPL;   // 16-byte value loads per lane
  uint4 k[2][4];     // key rows of tokens lane and 64 + lane (64 bytes each)
  uint4 v[NVI];      // value words, see gload_v
  uint16_t kmeta[4]; // lane i: scale[i], scale[i + 64], zero[i], zero[i + 64]
  float eb_c, eb_s;  // lane i: cos/sin(n Bk f_i)
  uint16_t vs[4], vz[4];  // value scale/zero of elements lane + 64 k ([group][token])
};

// Block pieces by slot g (slot_of); the rotary block base by position n.
__device__ __forceinline__ const uint8_t* gk_block(const kvq_cache& c, int64_t g) {
  return static_cast<const uint8_t*>(c.k_codes) + g * kBK * (kD / 2);
}
template <int VB>
__device__ __forceinline__ const uint8_t* gv_block(const kvq_cache& c, int64_t g) {
  constexpr int TPW = 32 / VB;
  return reinterpret_cast<const uint8_t*>(static_cast<const uint32_t*>(c.v_codes) + g * (kBK / TPW) * kD);
}
// Key row slot q (16 bytes) of half hf: token 64 hf + lane.
template <int VB>
__device__ __forceinline__ void gload_k(GRegs<VB>& R, int hf, int q, const uint8_t* kblk, int lane) {
  // plain loads: non-temporal ones made this kernel slower (c2 decode +3.6%), unlike the
  // one-head kernels
  R.k[hf][q] = *reinterpret_cast<const uint4*>(kblk + (uint32_t)((kHalf * hf + lane) * (kD / 2) + 16 * q));
}
// Value load s = (kc WPL + j) 2 + hc: word j of the 16 tokens 64 kc + 16 (lane / 16) ..
// of channels 64 hc + 4 (lane % 16) .. +3 (one word per channel).
template <int VB>
__device__ __forceinline__ void gload_v(GRegs<VB>& R, int s, const uint8_t* vblk, int lane) {
  constexpr int TPW = GRegs<VB>::TPW, WPL = GRegs<VB>::WPL;
  const int kc = s / (2 * WPL), j = (s >> 1) % WPL, hc = s & 1;
  const uint32_t tg = kc * (kHalf / TPW) + (lane >> 4) * WPL + j;
  R.v[s] = *reinterpret_cast<const uint4*>(vblk + (tg * kD + 64 * hc + 4 * (lane & 15)) * 4u);
}
template <int VB>
__device__ __forceinline__ void gload_kmeta(GRegs<VB>& R, const kvq_cache& c, int64_t g, int64_t n, int lane) {
  const int64_t m = g * kD;
  R.kmeta[0] = c.k_scale[m + lane];
  R.kmeta[1] = c.k_scale[m + lane + kHalf];
  R.kmeta[2] = c.k_zero[m + lane];
  R.kmeta[3] = c.k_zero[m + lane + kHalf];
  const float2 eb = reinterpret_cast<const float2*>(c.rope + (int64_t)kBK * kD + n * kD)[lane];
  R.eb_c = eb.x;
  R.eb_s = eb.y;
}
template <int VB>
__device__ __forceinline__ void gload_vmeta(GRegs<VB>& R, const kvq_cache& c, int64_t g, int lane, int ng) {
  const int64_t m0 = g * kBK * ng;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (kWave * k < kBK * ng) {
      const int grp = (kWave * k) / kBK, t = (kWave * k) % kBK + lane;
      const uint32_t e = (uint32_t)(t * ng + grp);
      R.vs[k] = c.v_scale[m0 + e];
      R.vz[k] = c.v_zero[m0 + e];
    }
  }
}

struct GState {
  float m[4], lpart[4], zpart[4][2];
  float acc[8];  // head lane / 16; channels 4 (lane % 16) + c (c < 4) and 64 + 4 (lane % 16) + c - 4
};

// Adds the value-outlier corrections (fixed point in LDS) of the lane's head and
// channels to its accumulators and clears them.
__device__ __forceinline__ void merge_vcorr_heads(int* VCI, GState& st, int lane) {
  const int hd = lane >> 4, c4 = 4 * (lane & 15);
  const int sh = VCI[4 * kD + hd];
#pragma unroll
  for (int hc = 0; hc < 2; ++hc) {
    int4* pc = reinterpret_cast<int4*>(VCI + hd * kD + 64 * hc + c4);
    const int4 v = *pc;
    st.acc[4 * hc] += __builtin_amdgcn_ldexpf((float)v.x, -sh);
    st.acc[4 * hc + 1] += __builtin_amdgcn_ldexpf((float)v.y, -sh);
    st.acc[4 * hc + 2] += __builtin_amdgcn_ldexpf((float)v.z, -sh);
    st.acc[4 * hc + 3] += __builtin_amdgcn_ldexpf((float)v.w, -sh);
    *pc = make_int4(0, 0, 0, 0);
  }
}

// Positions of the reduction index: the 16 bytes (4 dwords) a lane gives the integer
// MFMA for its 16 tokens are the code bytes in the order the packed words yield them,
// dword q byte m = token tau(q, m) of the 16: for 4-bit words (w & 0x0F0F0F0F, then
// (w >> 4) & ...) the even tokens of a word, then the odd; for 2-bit words
// ((w >> 2 q) & 0x03030303) tokens q, q + 4, q + 8, q + 12.
template <int VB>
__device__ __forceinline__ int tau(int q, int m) {
  return VB == 4 ? 8 * (q >> 1) + (q & 1) + 2 * m : q + 4 * m;
}

template <int VB, int KO, int NG, bool PG>
__device__ __forceinline__ void gqa_block(GRegs<VB>& R, CsrTok& C, GState& st, float* __restrict__ wl, const GLds& L,
                                          const float* __restrict__ table, int lane, int G, int ng,
                                          const kvq_cache& c, const SlotRow& sr, int64_t n, int nstep, bool more) {
  constexpr bool OUTL = KO > 0;
  constexpr int TPW = 32 / VB;
  const int64_t nn = more ? n + nstep : n;
  const int64_t gs = slot_at<PG>(sr, n), gnn = more ? slot_at<PG>(sr, nn) : gs;
  const uint8_t* knext = gk_block(c, gnn);
  const uint8_t* vnext = gv_block<VB>(c, gnn);
  float* Meta = wl + L.meta;
  float* WA = wl + L.wa;
  uint32_t* W32 = reinterpret_cast<uint32_t*>(wl + L.w32);  // [group][head][half][lane]
  int* VCI = reinterpret_cast<int*>(wl + L.vcorr);  // [4][D], then the 4 scale shifts
  const int hl = lane & 3;  // the head this lane feeds into the MFMA A operand
  const bool behind = behind_partner<kGqaWaves>(gqa_progress, lane);  // wave-uniform

  if (behind) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
  // value scale/zero and outlier entries of this block: needed only after the scores,
  // so they are loaded here rather than a block ahead.  Loads still in flight at the
  // block's end would be drained there (the counter is in order, so waiting for them
  // waits for the next block's code loads too).
  gload_vmeta(R, c, gs, lane, NG);
  if constexpr (OUTL) load_csr_tok<kBK, KO>(C, c, gs, lane);

  // ---- per-pair dequantization constants and block-rotated query weights (pair = lane)
  {
    // codes are read as fp16 subnormals (code_a * 2^-24, code_b * 2^-20): the scales
    // carry the inverse powers of two, so the products are exact as before
    const float sa = h2f(R.kmeta[0]) * 0x1p24f, sb = h2f(R.kmeta[1]) * 0x1p20f;
    *reinterpret_cast<float4*>(Meta + 4 * lane) = make_float4(sa, h2f(R.kmeta[2]), sb, h2f(R.kmeta[3]));
    const float4 q01 = *reinterpret_cast<const float4*>(wl + L.wq + 8 * lane);
    const float4 q23 = *reinterpret_cast<const float4*>(wl + L.wq + 8 * lane + 4);
    const float wq_r[4] = {q01.x, q01.z, q23.x, q23.z}, wq_i[4] = {q01.y, q01.w, q23.y, q23.w};
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float2*>(WA + g * kWAP + 2 * lane) =
          make_float2(wq_r[g] * R.eb_c - wq_i[g] * R.eb_s, -(wq_r[g] * R.eb_s + wq_i[g] * R.eb_c));  // W_r, -W_i
  }
  gload_kmeta(R, c, gnn, nn, lane);
  wave_lds_sync();

  // ---- scores: lane owns tokens lane and 64 + lane; per key channel and token half
  // one MFMA over the four heads.  Both tokens share each pair's constants and
  // weights; one 16-byte read covers two pairs of the table or of the weights.  The
  // loop runs over windows of two pairs and is software-pipelined: the LDS reads of
  // window w + 1 are issued before the arithmetic of window w.
  f4 S[2];
  {
    const float* trA = table + lane * kTP;
    const float* trB = table + (kHalf + lane) * kTP;
    const float* wal = WA + hl * kWAP;
    struct Win {
      float4 tA, tB, wa, M0, M1;  // cos/sin of both tokens, weights, pair constants
    };
    auto load_win = [&](int w, Win& L) {
      const int i = 2 * w;
      L.tA = *reinterpret_cast<const float4*>(trA + 2 * i);
      L.tB = *reinterpret_cast<const float4*>(trB + 2 * i);
      L.wa = *reinterpret_cast<const float4*>(wal + 2 * i);
      L.M0 = *reinterpret_cast<const float4*>(Meta + 4 * i);
      L.M1 = *reinterpret_cast<const float4*>(Meta + 4 * i + 4);
    };
    // two accumulator chains per half; an MFMA result is ready only about 40 cycles
    // after issue, so dependent MFMAs are kept four apart
    f4 sc[2][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) sc[hf][0] = sc[hf][1] = f4{0.f, 0.f, 0.f, 0.f};
    Win L[2];
    load_win(0, L[0]);
    uint32_t words[2][4];
    float ca[2][4], cb[2][4];
#pragma unroll
    for (int w = 0; w < kHalf / 2; ++w) {
      if (w % 8 == 0) {  // a new 16-byte slot of both rows; refill it with the next block
        const int q = w / 8;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          words[hf][0] = R.k[hf][q].x; words[hf][1] = R.k[hf][q].y;
          words[hf][2] = R.k[hf][q].z; words[hf][3] = R.k[hf][q].w;
          gload_k(R, hf, q, knext, lane);
        }
      }
      if (w % 2 == 0) {  // a new dword: pairs 4 d .. 4 d + 3, byte = (code_a | code_b << 4)
        const int d = (w % 8) / 2;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          // nibbles masked into bits 0-3 / 4-7 of a 16-bit half are exact fp16 subnormals,
          // read in place by the dequantizing FMAs (v_fma_mix_f32)
          const uint32_t x = words[hf][d], t = x >> 8;
          const h2t a02 = __builtin_bit_cast(h2t, x & 0x000F000Fu), b02 = __builtin_bit_cast(h2t, x & 0x00F000F0u);
          const h2t a13 = __builtin_bit_cast(h2t, t & 0x000F000Fu), b13 = __builtin_bit_cast(h2t, t & 0x00F000F0u);
          ca[hf][0] = (float)a02.x; ca[hf][1] = (float)a13.x; ca[hf][2] = (float)a02.y; ca[hf][3] = (float)a13.y;
          cb[hf][0] = (float)b02.x; cb[hf][1] = (float)b13.x; cb[hf][2] = (float)b02.y; cb[hf][3] = (float)b13.y;
        }
      }
      if (w + 1 < kHalf / 2) load_win(w + 1, L[(w + 1) & 1]);
      const Win& C0 = L[w & 1];
      const int m2 = 2 * (w % 2);
      float tr[2][2], ti[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4 M = u ? C0.M1 : C0.M0;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float4 t = hf ? C0.tB : C0.tA;
          const float cs = u ? t.z : t.x, sn = u ? t.w : t.y;
          const float ka = __builtin_fmaf(M.x, ca[hf][m2 + u], M.y);
          const float kb = __builtin_fmaf(M.z, cb[hf][m2 + u], M.w);
          tr[hf][u] = __builtin_fmaf(ka, cs, -(kb * sn));
          ti[hf][u] = __builtin_fmaf(ka, sn, kb * cs);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) sc[hf][u] = mfma4(u ? C0.wa.z : C0.wa.x, tr[hf][u], sc[hf][u]);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) sc[hf][u] = mfma4(u ? C0.wa.w : C0.wa.y, ti[hf][u], sc[hf][u]);
      // one window at a time: hoisting the reads of the whole unrolled block would
      // exhaust the registers
      __builtin_amdgcn_sched_barrier(0);
    }
    S[0] = sc[0][0] + sc[0][1];
    S[1] = sc[1][0] + sc[1][1];
  }

  // the block's serial part (softmax, value weights, value MFMAs, outliers) runs at a
  // raised wave priority, the score loop at the base one
  if (behind) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(1);

  // ---- online softmax per head; lane owns tokens lane and 64 + lane
  float p[2][4];
  float mloc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) mloc[g] = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int g = 0; g < 4; ++g) p[k][g] = S[k][g];
    if constexpr (OUTL) {
      // key outliers of token t: code 0 (dequantized to the zero-point) was stored; add
      // the exact term (x - zero) of each CSR entry, rotated, for every head
      const int t = kHalf * k + lane;
#pragma unroll
      for (int qq = 0; qq < KO; ++qq) {
        const int col = (int)((C.kc[k] >> (8 * qq)) & 0xffu);
        const float val = h2f((uint16_t)(C.kv[k] >> (16 * qq)));
        const int i = col % kHalf;
        const bool a = col < kHalf;
        const float4 M = *reinterpret_cast<const float4*>(Meta + 4 * i);
        const float dl = val - (a ? M.y : M.w);
        const float2 cssn = *reinterpret_cast<const float2*>(table + t * kTP + 2 * i);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float2 w = *reinterpret_cast<const float2*>(WA + g * kWAP + 2 * i);
          const float wr = w.x, wi = -w.y;
          const float re = wr * cssn.x - wi * cssn.y, im = wr * cssn.y + wi * cssn.x;
          p[k][g] += a ? dl * re : -dl * im;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) mloc[g] = fmaxf(mloc[g], p[k][g]);
  }
  if constexpr (OUTL) merge_vcorr_heads(VCI, st, lane);  // the previous block's, before the rescale
  const int hd = lane >> 4;  // the head of the lane's value accumulators
  float pmax[4], alpha_hd = 0.0f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float mb = wave_max_uniform(mloc[g]);
    const float mnew = fmaxf(st.m[g], mb);
    const float alpha = __builtin_amdgcn_exp2f(st.m[g] - mnew);
    st.m[g] = mnew;
    pmax[g] = __builtin_amdgcn_exp2f(mb - mnew);  // the p of the block's top token
    p[0][g] = __builtin_amdgcn_exp2f(p[0][g] - mnew);
    p[1][g] = __builtin_amdgcn_exp2f(p[1][g] - mnew);
    st.lpart[g] = __builtin_fmaf(st.lpart[g], alpha, p[0][g] + p[1][g]);
    alpha_hd = hd == g ? alpha : alpha_hd;
    st.zpart[g][0] *= alpha;
    st.zpart[g][1] *= alpha;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] *= alpha_hd;

  // ---- value weights w = p * scale of [group][head][token] in 30-bit fixed point: the
  // weights of head g and group k are at most bound = pmax_g * (the block's largest
  // scale of group k), so W = rint(w 2^30 / bound) <= 2^30 (1 + 2^-21).  W is stored as
  // four balanced base-256 digits d_r in [-128, 127], W = sum_r d_r 256^r: the bytes of
  // (W + 0x80808080) ^ 0x80808080 read as int8 (exact for W < 0x7F7F7F80).  Each weight
  // is then exact up to half a unit (2^-31 bound) and the fp32 rounding of w 2^30 / bound,
  // and the integer products below are exact; the zero-point part p * zero is summed
  // per lane in fp32.  Element lane + 64 k is token 64 (k % 2) + lane of group k / 2.
  float vzc[4] = {0.f, 0.f, 0.f, 0.f}, inv_hd[2] = {0.f, 0.f};
  {
    float vsf[4], vmax[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2 * NG; ++k) {
      vsf[k] = h2f(R.vs[k]);
      vzc[k] = h2f(R.vz[k]);
      vmax[k >> 1] = fmaxf(vmax[k >> 1], vsf[k]);
    }
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      vmax[grp] = wave_max_uniform(vmax[grp]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float bound = pmax[g] * vmax[grp];
        const float kq = bound > 0x1p-100f ? 0x1p30f * __builtin_amdgcn_rcpf(bound) : 0.0f;
        const uint32_t w0 = (uint32_t)__builtin_rintf(p[0][g] * vsf[2 * grp] * kq);
        const uint32_t w1 = (uint32_t)__builtin_rintf(p[1][g] * vsf[2 * grp + 1] * kq);
        W32[((grp * 4 + g) * 2) * kW32P + lane] = (w0 + 0x80808080u) ^ 0x80808080u;
        W32[((grp * 4 + g) * 2 + 1) * kW32P + lane] = (w1 + 0x80808080u) ^ 0x80808080u;
        st.zpart[g][grp] = __builtin_fmaf(p[0][g], vzc[2 * grp], __builtin_fmaf(p[1][g], vzc[2 * grp + 1], st.zpart[g][grp]));
        inv_hd[grp] = hd == g ? bound * 0x1p-30f : inv_hd[grp];
      }
    }
  }
  wave_lds_sync();

  // ---- values: D[(head, digit)][channel] += sum over 64 tokens of digit * code, per
  // token half kc and channel tile T (channels 64 (T / 4) + 4 (lane % 16) + T % 4)
  {
    constexpr int WPL = GRegs<VB>::WPL;
    // A: row lane % 16 = (head h_a, digit pl), tokens 16 (lane / 16) + tau(q, m) of each
    // half: byte pl of the tokens' digit words, gathered four at a time by v_perm
    const int h_a = (lane >> 2) & 3, pl = lane & 3, lg = lane >> 4;
    const uint32_t sel = (uint32_t)pl | ((uint32_t)(4 + pl) << 8) | 0x0C0C0000u;  // byte pl of S1, of S0, zeros
    i4 A[2][NG];
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const uint4* wr = reinterpret_cast<const uint4*>(W32 + ((grp * 4 + h_a) * 2 + kc) * kW32P + 16 * lg);
        uint32_t x[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 e = wr[u];
          x[4 * u] = e.x; x[4 * u + 1] = e.y; x[4 * u + 2] = e.z; x[4 * u + 3] = e.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t ab = __builtin_amdgcn_perm(x[tau<VB>(q, 1)], x[tau<VB>(q, 0)], sel);
          const uint32_t cd = __builtin_amdgcn_perm(x[tau<VB>(q, 3)], x[tau<VB>(q, 2)], sel);
          A[kc][grp][q] = (int)__builtin_amdgcn_perm(cd, ab, 0x05040100u);
        }
      }
    }
    i4 Dt[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) Dt[t] = i4{0, 0, 0, 0};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          i4 B;
          if constexpr (VB == 4) {
            const uint4 va = R.v[(kc * WPL) * 2 + hc], vb = R.v[(kc * WPL + 1) * 2 + hc];
            const uint32_t wa = t4 == 0 ? va.x : t4 == 1 ? va.y : t4 == 2 ? va.z : va.w;
            const uint32_t wb = t4 == 0 ? vb.x : t4 == 1 ? vb.y : t4 == 2 ? vb.z : vb.w;
            B = i4{(int)(wa & 0x0F0F0F0Fu), (int)((wa >> 4) & 0x0F0F0F0Fu), (int)(wb & 0x0F0F0F0Fu),
                   (int)((wb >> 4) & 0x0F0F0F0Fu)};
          } else {
            const uint4 va = R.v[kc * 2 + hc];
            const uint32_t w = t4 == 0 ? va.x : t4 == 1 ? va.y : t4 == 2 ? va.z : va.w;
            B = i4{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
                   (int)((w >> 6) & 0x03030303u)};
          }
          Dt[4 * hc + t4] = mfma_i8(A[kc][NG == 2 ? hc : 0], B, Dt[4 * hc + t4]);
        }
#pragma unroll
        for (int j = 0; j < WPL; ++j) gload_v(R, (kc * WPL + j) * 2 + hc, vnext, lane);
      }
    }
    // lane holds rows 4 hd + r (digit r of head hd) of its channel in every tile; a row
    // sum is at most 128 x 128 x 15 in magnitude (the top digit's at most 128 x 64 x 15),
    // so the digit pairs combine exactly in 32 bits before the fp32 conversion
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int hi = Dt[t][3] * 256 + Dt[t][2], lo = Dt[t][1] * 256 + Dt[t][0];
      const float inv = inv_hd[NG == 2 ? t >> 2 : 0];
      st.acc[t] = __builtin_fmaf((float)hi, inv * 65536.0f, __builtin_fmaf((float)lo, inv, st.acc[t]));
    }
  }

  // ---- value outliers: p * (x - zero) scattered into the per-head channel array in
  // fixed point; merged at the next block's softmax (or the item's end)
  if constexpr (OUTL) {
    float cr[2][KO][4];
    int col[2][KO];
    float csum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int qq = 0; qq < KO; ++qq) {
        col[k][qq] = (int)((C.vc[k] >> (8 * qq)) & 0xffu);
        const float dl = h2f((uint16_t)(C.vv[k] >> (16 * qq))) - (col[k][qq] >= G ? vzc[2 + k] : vzc[k]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          cr[k][qq][g] = p[k][g] * dl;
          csum[g] += fabsf(cr[k][qq][g]);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int sh = vcorr_shift(wave_sum_uniform(csum[g]));
      if (lane == 0) VCI[4 * kD + g] = sh;
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int qq = 0; qq < KO; ++qq) atomicAdd(VCI + g * kD + col[k][qq], vcorr_fixed(cr[k][qq][g], sh));
    }
  }
  wave_lds_sync();
}

// Item = (b, kv-head, head set, split): the wave serves GW (4 or 2) query heads of the
// group; with 2 the MFMA rows of heads 2 and 3 carry zero weights.
template <int VB, int GW, int KO, int NG, bool PG>
__global__ __launch_bounds__(kGqaWaves * 64) void decode_gqa_kernel(kvq_cache c, const uint16_t* __restrict__ q,
                                                                   int64_t q_pos, float* __restrict__ ws, int S,
                                                                   int64_t nitems, const SeqOrder ord) {
  constexpr int kNT = kGqaWaves * 64;
  constexpr bool OUTL = KO > 0;
  extern __shared__ float lds[];
  const int H = c.cfg.kv_heads, Hq = c.cfg.q_heads, gq = Hq / H, nsets = gq / GW;
  const int G = c.cfg.v_group;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  float* table = lds;
  for (int idx = threadIdx.x; idx < kBK * kHalf; idx += kNT) {
    const int j = idx / kHalf, i = idx % kHalf;
    *reinterpret_cast<float2*>(table + j * kTP + 2 * i) = *reinterpret_cast<const float2*>(c.rope + 2 * idx);
  }
  const GLds L = gqa_lds(NG, OUTL);
  float* wl = lds + kBK * kTP + wave * L.total;
  if (OUTL)
    for (int k = lane; k < 4 * kD + 4; k += kWave) reinterpret_cast<int*>(wl + L.vcorr)[k] = 0;
  if (threadIdx.x < kGqaWaves) gqa_progress[threadIdx.x] = 0;
  __syncthreads();

  const int64_t total_waves = (int64_t)gridDim.x * kGqaWaves;
  const int64_t p = (int64_t)blockIdx.x * kGqaWaves + wave;
  const int64_t per_seq = (int64_t)H * nsets * S;
  // per-sequence lengths: items in length order, dealt in a snake (every wave exits once
  // k passes nitems); dense: item p, p + total_waves, ...
  for (int64_t r = 0;; ++r) {
    const int64_t k = PG ? snake_item(r, p, total_waves) : p + r * total_waves;
    if (k >= nitems) break;
    const int64_t item = PG ? ordered_item(ord, k, per_seq) : k;
    const int split = (int)(item % S);
    const int64_t rest = item / S;
    const int set = (int)(rest % nsets);
    const int64_t bh = rest / nsets;
    const int h = (int)(bh % H);
    const int b = (int)(bh / H);
    // the sequence's own length and newest position in a cache with per-sequence lengths
    const int64_t len_b = seq_len_t<PG>(c, b);
    const int64_t nfull = len_b / kBK;
    const int64_t qp = q_pos < 0 ? len_b - 1 : q_pos;
    // split `split` takes blocks split, split + S, ...: the waves of a workgroup hold
    // consecutive splits, so together they stream neighbouring blocks
    const int64_t n0 = split;

    // query weights of pair `lane` per head: scale * conj(q_g,i) e^{-i f_i q_pos} (fp64)
    float wq_r[4], wq_i[4];
    {
      const double f = pow((double)c.cfg.rope_theta, -(2.0 * lane) / (double)kD);
      double sn, cs;
      sincos((double)qp * f, &sn, &cs);
      const double scl = (double)kLog2e / sqrt((double)kD);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        wq_r[g] = 0.0f;
        wq_i[g] = 0.0f;
        if (g < GW) {
          const int hq = h * gq + set * GW + g;
          const uint16_t* qv = q + ((int64_t)b * Hq + hq) * kD;
          const double qa = (double)h2f(qv[lane]), qb = (double)h2f(qv[lane + kHalf]);
          wq_r[g] = (float)(scl * (qa * cs - qb * sn));
          wq_i[g] = (float)(-scl * (qa * sn + qb * cs));
        }
      }
      *reinterpret_cast<float4*>(wl + L.wq + 8 * lane) = make_float4(wq_r[0], wq_i[0], wq_r[1], wq_i[1]);
      *reinterpret_cast<float4*>(wl + L.wq + 8 * lane + 4) = make_float4(wq_r[2], wq_i[2], wq_r[3], wq_i[3]);
      wave_lds_sync();
    }
    GState st;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      st.m[g] = -__builtin_inff();
      st.lpart[g] = 0.0f;
      st.zpart[g][0] = st.zpart[g][1] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[t] = 0.0f;

    GRegs<VB> R;
    CsrTok C;
    const SlotRow sr = slot_row(c, b, h);
    if (n0 < nfull) {
      const int64_t g0 = slot_at<PG>(sr, n0);
      gload_kmeta(R, c, g0, n0, lane);
      const uint8_t* kb0 = gk_block(c, g0);
      const uint8_t* vb0 = gv_block<VB>(c, g0);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) gload_k(R, hf, qq, kb0, lane);
#pragma unroll
      for (int s = 0; s < GRegs<VB>::NVI; ++s) gload_v(R, s, vb0, lane);
    }
    for (int64_t n = n0; n < nfull; n += S)
      gqa_block<VB, KO, NG, PG>(R, C, st, wl, L, table, lane, G, NG, c, sr, n, S, n + S < nfull);

    if (OUTL) {  // the item's last block of value corrections
      merge_vcorr_heads(reinterpret_cast<int*>(wl + L.vcorr), st, lane);
      wave_lds_sync();
    }
    // ---- finish the item: (m, l) per head from lane 0, o from the 16 lanes of its head
    float zl[2] = {0.f, 0.f};
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float l = wave_sum(st.lpart[g]);
      const float z0 = wave_sum(st.zpart[g][0]);
      const float z1 = NG == 2 ? wave_sum(st.zpart[g][1]) : 0.0f;
      zl[0] = (lane >> 4) == g ? z0 : zl[0];
      zl[1] = (lane >> 4) == g ? z1 : zl[1];
      if (lane == 0) {
        float* dst = ws + (((int64_t)b * Hq + h * gq + set * GW + g) * S + split) * (kD + 2);
        dst[0] = st.m[g];
        dst[1] = l;
      }
    }
    const int hd = lane >> 4;
    if (hd < GW) {
      float* dst = ws + (((int64_t)b * Hq + h * gq + set * GW + hd) * S + split) * (kD + 2);
      const int c4 = 4 * (lane & 15);
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) {
        const float z = NG == 2 && hc == 1 ? zl[1] : zl[0];  // channels 64 hc + c4 .. lie in group hc when G = 64
        *reinterpret_cast<float4*>(dst + 2 + 64 * hc + c4) =
            make_float4(st.acc[4 * hc] + z, st.acc[4 * hc + 1] + z, st.acc[4 * hc + 2] + z, st.acc[4 * hc + 3] + z);
      }
    }
  }
}

template <int VB, int GW, int KO, int NG, bool PG>
hipError_t launch_gqa_typed(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S, hipStream_t s,
                            int cus, bool dry) {
  const GLds L = gqa_lds(NG, KO > 0);
  const size_t bytes = ((size_t)kBK * kTP + (size_t)kGqaWaves * L.total) * sizeof(float);
  if (bytes + kGqaWaves * sizeof(int) > 160 * 1024) return hipErrorNotSupported;  // with the static progress counts
  if (dry) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)decode_gqa_kernel<VB, GW, KO, NG, PG>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  const int gq = c.cfg.q_heads / c.cfg.kv_heads;
  const int64_t nitems = (int64_t)c.cfg.batch * c.cfg.kv_heads * (gq / GW) * S;
  int64_t grid = (nitems + kGqaWaves - 1) / kGqaWaves;
  if (grid > cus) grid = cus;
  hipLaunchKernelGGL((decode_gqa_kernel<VB, GW, KO, NG, PG>), dim3((unsigned)grid), dim3(kGqaWaves * 64), bytes, s, c, q,
                     q_pos, ws, S, nitems, PG ? seq_order(c) : SeqOrder{0, {}});
  return hipGetLastError();
}

}  // namespace

// Returns hipErrorNotSupported when the configuration is not one this kernel covers; with
// `dry` it launches nothing and only reports whether it does.
hipError_t launch_decode_gqa(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S,
                             hipStream_t s, int cus, bool dry) {
  const kvq_config& g = c.cfg;
  const int ko = host_kout(g);
  const int gq = g.q_heads / g.kv_heads;
  const int ng = g.head_dim / g.v_group;
  if (gq < 2 || gq % 2 || g.k_mode != 0 || g.k_bits != 4 || ko > 2 || ng < 1 || ng > 2 || g.head_dim != kD ||
      g.k_block != kBK || (g.v_bits != 4 && g.v_bits != 2) || g.keep_pct > 0 || g.v_mode != 0)
    return hipErrorNotSupported;
  const bool four = gq % 4 == 0;
  // per-sequence lengths (dense or paged slots): a kernel of their own
#define KVQ_GQA_NG(vb, gw, ko)                                                                     \
  if (c.seq_lens)                                                                                  \
    return ng == 2 ? launch_gqa_typed<vb, gw, ko, 2, true>(c, q, q_pos, ws, S, s, cus, dry)         \
                   : launch_gqa_typed<vb, gw, ko, 1, true>(c, q, q_pos, ws, S, s, cus, dry);        \
  return ng == 2 ? launch_gqa_typed<vb, gw, ko, 2, false>(c, q, q_pos, ws, S, s, cus, dry)          \
                 : launch_gqa_typed<vb, gw, ko, 1, false>(c, q, q_pos, ws, S, s, cus, dry);
#define KVQ_GQA(vb, gw)                                                                       \
  if (g.v_bits == vb && four == (gw == 4)) {                                                  \
    if (ko == 2) { KVQ_GQA_NG(vb, gw, 2) }                                                    \
    if (ko == 1) { KVQ_GQA_NG(vb, gw, 1) }                                                    \
    KVQ_GQA_NG(vb, gw, 0)                                                                     \
  }
  KVQ_GQA(4, 4) KVQ_GQA(2, 4) KVQ_GQA(4, 2) KVQ_GQA(2, 2)
#undef KVQ_GQA
#undef KVQ_GQA_NG
  return hipErrorNotSupported;
}

}  // namespace kvq
