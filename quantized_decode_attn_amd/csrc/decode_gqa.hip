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
//  * values: lane l owns channels 4 (l % 32) .. +3 and the token groups of its half
//    of the wave; per token and channel slot one MFMA multiplies the four heads'
//    weights p * scale with the codes (converted two at a time with the packed fp8
//    conversion: a byte 0..15 is an exact fp8 value proportional to it);
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
constexpr int kD = 128, kBK = 128, kHalf = 64;
constexpr int kTP = kD + 4;  // floats per rotary-table row: 64 (cos, sin) pairs + 4 (banks)
constexpr int kWVP = kBK + 4;  // floats per value-weight row (one row per group and head)

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// Per-wave LDS area, in floats.
struct GLds {
  int meta, wa, wv, vcorr, wq, total;
};
__host__ __device__ inline GLds gqa_lds(int ng, bool outl) {
  GLds m;
  int o = 0;
  m.meta = o; o += 4 * kHalf;        // per pair: scale_a / u, zero_a, scale_b / u, zero_b
  m.wa = o; o += 4 * kHalf * 2;      // per head and pair: (W_r, -W_i)
  m.wv = o; o += ng * 4 * kWVP;      // value weights p * scale / u, [group][head][token]
  m.vcorr = o; o += outl ? 4 * kD + 4 : 0;  // value outlier corrections [head][channel] (int), scale per head
  m.wq = o; o += kHalf * 8;          // the item's query weights per pair: (re, im) of 4 heads
  m.total = o;
  return m;
}

template <int VB>
struct GRegs {
  static constexpr int NVI = (kBK / (32 / VB)) * kD / 256;  // 16-byte value loads per lane
  uint4 k[2][4];     // key rows of tokens lane and 64 + lane (64 bytes each)
  uint4 v[NVI];      // value words: load s holds channels 4 (l % 32) .. +3 of token group 2 s + l / 32
  uint16_t kmeta[4]; // lane i: scale[i], scale[i + 64], zero[i], zero[i + 64]
  float eb_c, eb_s;  // lane i: cos/sin(n Bk f_i)
  uint16_t vs[4], vz[4];  // value scale/zero of elements lane + 64 k ([group][token])
};

__device__ __forceinline__ const uint8_t* gk_block(const kvq_cache& c, int64_t bh, int64_t n) {
  return static_cast<const uint8_t*>(c.k_codes) + (bh * c.cfg.capacity + n * kBK) * (kD / 2);
}
template <int VB>
__device__ __forceinline__ const uint8_t* gv_block(const kvq_cache& c, int64_t bh, int64_t n) {
  constexpr int TPW = 32 / VB;
  return reinterpret_cast<const uint8_t*>(static_cast<const uint32_t*>(c.v_codes) +
                                          (bh * (c.cfg.capacity / TPW) + n * (kBK / TPW)) * kD);
}
// Key row slot q (16 bytes) of half hf: token 64 hf + lane.
template <int VB>
__device__ __forceinline__ void gload_k(GRegs<VB>& R, int hf, int q, const uint8_t* kblk, int lane) {
  R.k[hf][q] = *reinterpret_cast<const uint4*>(kblk + (uint32_t)((kHalf * hf + lane) * (kD / 2) + 16 * q));
}
// Value load s: words of token group 2 s + lane / 32 (32 / VB tokens each), channels
// 4 (lane % 32) .. +3.
template <int VB>
__device__ __forceinline__ void gload_v(GRegs<VB>& R, int s, const uint8_t* vblk, int lane) {
  const uint32_t tg = 2 * s + (lane >> 5);
  R.v[s] = *reinterpret_cast<const uint4*>(vblk + (tg * kD + 4 * (lane & 31)) * 4u);
}
template <int VB>
__device__ __forceinline__ void gload_kmeta(GRegs<VB>& R, const kvq_cache& c, int64_t bh, int64_t n, int lane) {
  const int64_t m = (bh * (c.cfg.capacity / kBK) + n) * kD;
  R.kmeta[0] = c.k_scale[m + lane];
  R.kmeta[1] = c.k_scale[m + lane + kHalf];
  R.kmeta[2] = c.k_zero[m + lane];
  R.kmeta[3] = c.k_zero[m + lane + kHalf];
  const float2 eb = reinterpret_cast<const float2*>(c.rope + (int64_t)kBK * kD + n * kD)[lane];
  R.eb_c = eb.x;
  R.eb_s = eb.y;
}
template <int VB>
__device__ __forceinline__ void gload_vmeta(GRegs<VB>& R, const kvq_cache& c, int64_t bh, int64_t n, int lane,
                                            int ng) {
  const int64_t m0 = (bh * c.cfg.capacity + n * kBK) * ng;
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
  f4 acc[4];  // acc[c][g]: head g, channel 4 (lane % 32) + c, this lane's token groups
};

// Adds the four heads' value-outlier corrections (fixed point in LDS) to the lane's
// accumulators (channels 4 lane .. +3, lanes < 32) and clears them.
__device__ __forceinline__ void merge_vcorr_heads(int* VCI, GState& st, int lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float a[4] = {st.acc[0][g], st.acc[1][g], st.acc[2][g], st.acc[3][g]};
    merge_vcorr<kD>(VCI + g * kD, VCI[4 * kD + g], a, lane);
    st.acc[0][g] = a[0]; st.acc[1][g] = a[1]; st.acc[2][g] = a[2]; st.acc[3][g] = a[3];
  }
}

template <int VB, int KO>
__device__ __forceinline__ void gqa_block(GRegs<VB>& R, CsrTok& C, GState& st, float* __restrict__ wl, const GLds& L,
                                          const float* __restrict__ table, float inv_unit, int lane, int G, int ng,
                                          const kvq_cache& c, int64_t bh, int64_t n, bool more) {
  constexpr bool OUTL = KO > 0;
  constexpr int TPW = 32 / VB;
  const int64_t nn = more ? n + 1 : n;
  const uint8_t* knext = gk_block(c, bh, nn);
  const uint8_t* vnext = gv_block<VB>(c, bh, nn);
  float* Meta = wl + L.meta;
  float* WA = wl + L.wa;
  float* WV = wl + L.wv;
  int* VCI = reinterpret_cast<int*>(wl + L.vcorr);  // [4][D], then the 4 scale shifts
  const int hl = lane & 3;  // the head this lane feeds into the MFMA A operand

  // ---- per-pair dequantization constants and block-rotated query weights (pair = lane)
  {
    const float sa = h2f(R.kmeta[0]) * inv_unit, sb = h2f(R.kmeta[1]) * inv_unit;
    *reinterpret_cast<float4*>(Meta + 4 * lane) = make_float4(sa, h2f(R.kmeta[2]), sb, h2f(R.kmeta[3]));
    const float4 q01 = *reinterpret_cast<const float4*>(wl + L.wq + 8 * lane);
    const float4 q23 = *reinterpret_cast<const float4*>(wl + L.wq + 8 * lane + 4);
    const float wq_r[4] = {q01.x, q01.z, q23.x, q23.z}, wq_i[4] = {q01.y, q01.w, q23.y, q23.w};
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float2*>(WA + g * 2 * kHalf + 2 * lane) =
          make_float2(wq_r[g] * R.eb_c - wq_i[g] * R.eb_s, -(wq_r[g] * R.eb_s + wq_i[g] * R.eb_c));  // W_r, -W_i
  }
  gload_kmeta(R, c, bh, nn, lane);
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
    const float* wal = WA + hl * 2 * kHalf;
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
          const uint32_t lo = words[hf][d] & 0x0F0F0F0Fu, hi = (words[hf][d] >> 4) & 0x0F0F0F0Fu;
          const f2v a01 = cvt_lo(lo), a23 = cvt_hi(lo), b01 = cvt_lo(hi), b23 = cvt_hi(hi);
          ca[hf][0] = a01.x; ca[hf][1] = a01.y; ca[hf][2] = a23.x; ca[hf][3] = a23.y;
          cb[hf][0] = b01.x; cb[hf][1] = b01.y; cb[hf][2] = b23.x; cb[hf][3] = b23.y;
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
          const float2 w = *reinterpret_cast<const float2*>(WA + g * 2 * kHalf + 2 * i);
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
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float mnew = fmaxf(st.m[g], wave_max_uniform(mloc[g]));
    const float alpha = __builtin_amdgcn_exp2f(st.m[g] - mnew);
    st.m[g] = mnew;
    p[0][g] = __builtin_amdgcn_exp2f(p[0][g] - mnew);
    p[1][g] = __builtin_amdgcn_exp2f(p[1][g] - mnew);
    st.lpart[g] = __builtin_fmaf(st.lpart[g], alpha, p[0][g] + p[1][g]);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) st.acc[cc][g] *= alpha;
    st.zpart[g][0] *= alpha;
    st.zpart[g][1] *= alpha;
  }

  // ---- value weights p * scale / u per [group][head][token] (the codes enter the
  // MFMA as c * u); the zero-point part p * zero is summed per lane in fp32.
  // Element lane + 64 k is token 64 (k % 2) + lane of group k / 2.
  float vzc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    vzc[k] = 0.0f;
    if (kWave * k < kBK * ng) {
      const int grp = k >> 1, kt = k & 1;
      const float vs = h2f(R.vs[k]) * inv_unit, vz = h2f(R.vz[k]);
      vzc[k] = vz;
      float* wvp = WV + grp * 4 * kWVP + kHalf * kt + lane;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        wvp[g * kWVP] = p[kt][g] * vs;
        st.zpart[g][grp] = __builtin_fmaf(p[kt][g], vz, st.zpart[g][grp]);
      }
    }
  }
  gload_vmeta(R, c, bh, nn, lane, ng);
  wave_lds_sync();

  // ---- values: per token and channel slot one MFMA over the four heads
  {
    f4 va[4];  // even-token chains; the odd tokens accumulate into st.acc directly
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) va[cc] = f4{0.f, 0.f, 0.f, 0.f};
    const int grp_l = (4 * (lane & 31)) / G;
    const float* wvl = WV + (grp_l * 4 + hl) * kWVP + TPW * (lane >> 5);
#pragma unroll
    for (int s = 0; s < GRegs<VB>::NVI; ++s) {
      const uint32_t words[4] = {R.v[s].x, R.v[s].y, R.v[s].z, R.v[s].w};
      gload_v(R, s, vnext, lane);
      float wt[TPW];  // weights of the group's tokens for head lane % 4
#pragma unroll
      for (int u4 = 0; u4 < TPW; u4 += 4) {
        const float4 x = *reinterpret_cast<const float4*>(wvl + 2 * TPW * s + u4);
        wt[u4] = x.x; wt[u4 + 1] = x.y; wt[u4 + 2] = x.z; wt[u4 + 3] = x.w;
      }
      // two channel slots at a time, each with an even-token and an odd-token chain,
      // so that four independent MFMA chains alternate
#pragma unroll
      for (int c2 = 0; c2 < 4; c2 += 2) {
        float cv[2][TPW];  // codes (times u) of the two words' tokens
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint32_t w = words[c2 + h2];
          if constexpr (VB == 4) {
            const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
            const f2v e0 = cvt_lo(lo), e1 = cvt_hi(lo), o0 = cvt_lo(hi), o1 = cvt_hi(hi);
            cv[h2][0] = e0.x; cv[h2][2] = e0.y; cv[h2][4] = e1.x; cv[h2][6] = e1.y;
            cv[h2][1] = o0.x; cv[h2][3] = o0.y; cv[h2][5] = o1.x; cv[h2][7] = o1.y;
          } else {
#pragma unroll
            for (int sh = 0; sh < 4; ++sh) {  // tokens sh, sh + 4, sh + 8, sh + 12
              const uint32_t x = (w >> (2 * sh)) & 0x03030303u;
              const f2v lo2 = cvt_lo(x), hi2 = cvt_hi(x);
              cv[h2][sh] = lo2.x; cv[h2][sh + 4] = lo2.y; cv[h2][sh + 8] = hi2.x; cv[h2][sh + 12] = hi2.y;
            }
          }
        }
#pragma unroll
        for (int u = 0; u < TPW; u += 2) {
          va[c2] = mfma4(wt[u], cv[0][u], va[c2]);
          va[c2 + 1] = mfma4(wt[u], cv[1][u], va[c2 + 1]);
          st.acc[c2] = mfma4(wt[u + 1], cv[0][u + 1], st.acc[c2]);
          st.acc[c2 + 1] = mfma4(wt[u + 1], cv[1][u + 1], st.acc[c2 + 1]);
        }
      }
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) st.acc[cc] += va[cc];
  }

  // ---- value outliers: p * (x - zero) scattered into the per-head channel array in
  // fixed point; merged at the next block's softmax (or the item's end)
  if constexpr (OUTL) {
    float cr[2][KO][4];
    int col[2][KO];
    float cmax[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int qq = 0; qq < KO; ++qq) {
        col[k][qq] = (int)((C.vc[k] >> (8 * qq)) & 0xffu);
        const float dl = h2f((uint16_t)(C.vv[k] >> (16 * qq))) - (col[k][qq] >= G ? vzc[2 + k] : vzc[k]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          cr[k][qq][g] = p[k][g] * dl;
          cmax[g] = fmaxf(cmax[g], fabsf(cr[k][qq][g]));
        }
      }
    }
    load_csr_tok<kBK, KO>(C, c, bh, nn, lane);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int sh = vcorr_shift(wave_max_uniform(cmax[g]));
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
template <int VB, int GW, int KO>
__global__ __launch_bounds__(kGqaWaves * 64) void decode_gqa_kernel(kvq_cache c, const uint16_t* __restrict__ q,
                                                                   int64_t q_pos, float* __restrict__ ws, int S,
                                                                   int64_t nitems) {
  constexpr int kNT = kGqaWaves * 64;
  constexpr bool OUTL = KO > 0;
  extern __shared__ float lds[];
  const int H = c.cfg.kv_heads, Hq = c.cfg.q_heads, gq = Hq / H, nsets = gq / GW;
  const int G = c.cfg.v_group, ng = kD / G;
  const int64_t nfull = c.length / kBK;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  float* table = lds;
  for (int idx = threadIdx.x; idx < kBK * kHalf; idx += kNT) {
    const int j = idx / kHalf, i = idx % kHalf;
    *reinterpret_cast<float2*>(table + j * kTP + 2 * i) = *reinterpret_cast<const float2*>(c.rope + 2 * idx);
  }
  const GLds L = gqa_lds(ng, OUTL);
  float* wl = lds + kBK * kTP + wave * L.total;
  if (OUTL)
    for (int k = lane; k < 4 * kD + 4; k += kWave) reinterpret_cast<int*>(wl + L.vcorr)[k] = 0;
  __syncthreads();

  const float inv_unit = 1.0f / cvt_lo(1u).x;  // the fp8 value of the byte 1 is a power of two
  const int64_t total_waves = (int64_t)gridDim.x * kGqaWaves;
  for (int64_t item = (int64_t)blockIdx.x * kGqaWaves + wave; item < nitems; item += total_waves) {
    const int split = (int)(item % S);
    const int64_t rest = item / S;
    const int set = (int)(rest % nsets);
    const int64_t bh = rest / nsets;
    const int h = (int)(bh % H);
    const int b = (int)(bh / H);
    const int64_t n0 = nfull * split / S, n1 = nfull * (split + 1) / S;

    // query weights of pair `lane` per head: scale * conj(q_g,i) e^{-i f_i q_pos} (fp64)
    float wq_r[4], wq_i[4];
    {
      const double f = pow((double)c.cfg.rope_theta, -(2.0 * lane) / (double)kD);
      double sn, cs;
      sincos((double)q_pos * f, &sn, &cs);
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
      st.acc[g] = f4{0.f, 0.f, 0.f, 0.f};
    }

    GRegs<VB> R;
    CsrTok C;
    if (n0 < n1) {
      gload_kmeta(R, c, bh, n0, lane);
      gload_vmeta(R, c, bh, n0, lane, ng);
      if constexpr (OUTL) load_csr_tok<kBK, KO>(C, c, bh, n0, lane);
      const uint8_t* kb0 = gk_block(c, bh, n0);
      const uint8_t* vb0 = gv_block<VB>(c, bh, n0);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) gload_k(R, hf, qq, kb0, lane);
#pragma unroll
      for (int s = 0; s < GRegs<VB>::NVI; ++s) gload_v(R, s, vb0, lane);
    }
    for (int64_t n = n0; n < n1; ++n)
      gqa_block<VB, KO>(R, C, st, wl, L, table, inv_unit, lane, G, ng, c, bh, n, n + 1 < n1);

    if (OUTL) {  // the item's last block of value corrections
      merge_vcorr_heads(reinterpret_cast<int*>(wl + L.vcorr), st, lane);
      wave_lds_sync();
    }
    // ---- finish the item: the two token halves of each channel, then (m, l, o) per head
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int g = 0; g < 4; ++g) st.acc[cc][g] += __shfl_xor(st.acc[cc][g], 32, kWave);
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float l = wave_sum(st.lpart[g]);
      const float z0 = wave_sum(st.zpart[g][0]);
      const float z1 = wave_sum(st.zpart[g][1]);
      const int hq = h * gq + set * GW + g;
      float* dst = ws + (((int64_t)b * Hq + hq) * S + split) * (kD + 2);
      if (lane < 32) {
        const int ch0 = 4 * lane;
        const float z = (ch0 / G) == 0 ? z0 : z1;
        *reinterpret_cast<float4*>(dst + 2 + ch0) =
            make_float4(st.acc[0][g] + z, st.acc[1][g] + z, st.acc[2][g] + z, st.acc[3][g] + z);
      }
      if (lane == 0) {
        dst[0] = st.m[g];
        dst[1] = l;
      }
    }
  }
}

template <int VB, int GW, int KO>
hipError_t launch_gqa_typed(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S, hipStream_t s,
                            int cus) {
  const int ng = kD / c.cfg.v_group;
  const GLds L = gqa_lds(ng, KO > 0);
  const size_t bytes = ((size_t)kBK * kTP + (size_t)kGqaWaves * L.total) * sizeof(float);
  if (bytes > 160 * 1024) return hipErrorNotSupported;
  hipError_t e = hipFuncSetAttribute((const void*)decode_gqa_kernel<VB, GW, KO>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  const int gq = c.cfg.q_heads / c.cfg.kv_heads;
  const int64_t nitems = (int64_t)c.cfg.batch * c.cfg.kv_heads * (gq / GW) * S;
  int64_t grid = (nitems + kGqaWaves - 1) / kGqaWaves;
  if (grid > cus) grid = cus;
  hipLaunchKernelGGL((decode_gqa_kernel<VB, GW, KO>), dim3((unsigned)grid), dim3(kGqaWaves * 64), bytes, s, c, q,
                     q_pos, ws, S, nitems);
  return hipGetLastError();
}

}  // namespace

// Returns hipErrorNotSupported when the configuration is not one this kernel covers.
hipError_t launch_decode_gqa(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S,
                             hipStream_t s, int cus) {
  const kvq_config& g = c.cfg;
  const int ko = host_kout(g);
  const int gq = g.q_heads / g.kv_heads;
  const int ng = g.head_dim / g.v_group;
  if (gq < 2 || gq % 2 || g.k_mode != 0 || g.k_bits != 4 || ko > 2 || ng > 2 || g.head_dim != kD ||
      g.k_block != kBK || (g.v_bits != 4 && g.v_bits != 2))
    return hipErrorNotSupported;
  const bool four = gq % 4 == 0;
#define KVQ_GQA(vb, gw)                                                                       \
  if (g.v_bits == vb && four == (gw == 4)) {                                                  \
    if (ko == 2) return launch_gqa_typed<vb, gw, 2>(c, q, q_pos, ws, S, s, cus);              \
    if (ko == 1) return launch_gqa_typed<vb, gw, 1>(c, q, q_pos, ws, S, s, cus);              \
    return launch_gqa_typed<vb, gw, 0>(c, q, q_pos, ws, S, s, cus);                           \
  }
  KVQ_GQA(4, 4) KVQ_GQA(2, 4) KVQ_GQA(4, 2) KVQ_GQA(2, 2)
#undef KVQ_GQA
  return hipErrorNotSupported;
}

}  // namespace kvq
