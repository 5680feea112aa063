// decode_gqa.hip -- decode attention over uniform 2/4-bit key and value caches when
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
// rotation.  khat is computed once per key element and shared by every head of the
// group (6 operations per rotary pair, then 2 per head), unlike the one-head kernel,
// which folds the dequantization into per-head weights.
//
// Organisation (one wave per (b, kv-head, head set, split) item, blocks streamed
// through a register prefetch exactly as in the one-head kernel):
//  * per block, lanes < D/2 build the per-pair dequantization constants and the
//    block-rotated query weights of the wave's heads in LDS; every lane then holds
//    those of its 4 pairs in registers (16 lanes per key token);
//  * scores of all heads, reduced across a token's lanes by a DPP reduce-scatter
//    over the heads, written to LDS;
//  * outliers ([KVC3] "Per-Vector Dense-and-Sparse Quantization"): code 0 was stored
//    at an outlier's position; the lanes that own a token in the softmax (two tokens
//    per lane) add each of its CSR entries' exact score terms in registers, and
//    scatter its value corrections p * (x - zero) into a per-head channel array with
//    LDS atomics;
//  * online softmax per head over the block (lanes own two tokens each), value
//    weights p*scale quantized per head to 16-bit fixed point, nibble planes, and
//    v_dot8_u32_u4 on the packed value words as in the one-head kernel.
// No dequantized key or value is written to memory ([TQ] sections 5.1 and 6.3).
#include <math.h>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dcm;

constexpr int kGqaWaves = 8;
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// Per-wave LDS area, in floats.
struct GLds {
  int wts, s, vcorr, total;
};
__host__ __device__ inline GLds gqa_lds(int D, int BK, int GW, int ng, bool outl) {
  GLds m;
  int o = 0;
  const int wts = (4 + 2 * GW) * (D / 2);            // ALPHA BETA ZA ZB, then per pair WR[g] WIN[g]
  const int vq = GW * ng * BK / 2 + GW * ng * 64;     // u16 weights + nibble planes (reuse)
  m.wts = o; o += wts > vq ? wts : vq;
  m.s = o; o += BK * GW;                              // scores, then probabilities [BK][GW]
  m.vcorr = o; o += outl ? GW * D : 0;                // value outlier corrections [GW][D]
  m.total = o;
  return m;
}

// v + x of the DPP partner: row_mirror (lane 15 - i) and row_half_mirror (lane 7 - i).
__device__ __forceinline__ float add_dpp_rm(float v, float x) {
  asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %0 row_mirror row_mask:0xf bank_mask:0xf" : "+v"(v) : "v"(x));
  return v;
}
__device__ __forceinline__ float add_dpp_hm(float v, float x) {
  asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %0 row_half_mirror row_mask:0xf bank_mask:0xf" : "+v"(v) : "v"(x));
  return v;
}

template <int GW>
struct GState {
  float m[GW], lpart[GW], acc[GW][4], zpart[GW][2];
};

template <int D, int BK, int KB, int VB>
using GShape = MShape<D, BK, KB, VB, 4>;
template <int D, int BK, int KB, int VB>
using GRegs = BlockRegs<D, BK, KB, VB, GShape<D, BK, KB, VB>::NIT / 2, 4>;

template <int D, int BK, int KB, int VB, int GW, int KO>
__device__ __forceinline__ void gqa_block(GRegs<D, BK, KB, VB>& R, CsrTok& C, GState<GW>& st, float* __restrict__ wl,
                                          const GLds& L, const float* __restrict__ table, const float (&wq_r)[GW],
                                          const float (&wq_i)[GW], float unit, float inv_unit, int lane, int ts, int r, int G,
                                          int ng, const kvq_cache& c, int64_t bh, int64_t n, bool more,
                                          uint32_t koff) {
  using Sh = GShape<D, BK, KB, VB>;
  constexpr int HALF = Sh::HALF;
  constexpr bool OUTL = KO > 0;
  constexpr int ko = KO;
  const int64_t nn = more ? n + 1 : n;
  const uint8_t* knext = k_block<D, BK, KB, VB>(c, bh, nn);
  const uint8_t* vnext = v_block<D, BK, KB, VB>(c, bh, nn);
  float* wAL = wl + L.wts;
  float* wBE = wAL + HALF;
  float* wZA = wBE + HALF;
  float* wZB = wZA + HALF;
  float* wWP = wZB + HALF;        // [HALF][2 GW]: WR[g] then -WI[g] of each pair
  float* Sc = wl + L.s;           // [BK][GW]
  float* VCR = wl + L.vcorr;

  // ---- per-pair dequantization constants and block-rotated query weights
  // The codes arrive as c * u (u the fp8 unit, a power of two): keys are carried as
  // k * u = scale * (c u) + zero * u and the weights as W / u, which is exact scaling.
  if (lane < HALF) {
    reinterpret_cast<uint16_t*>(wAL)[lane] = R.kmeta[0];
    reinterpret_cast<uint16_t*>(wBE)[lane] = R.kmeta[1];
    wZA[lane] = h2f(R.kmeta[2]) * unit;
    wZB[lane] = h2f(R.kmeta[3]) * unit;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      wWP[lane * 2 * GW + g] = (wq_r[g] * R.eb_c - wq_i[g] * R.eb_s) * inv_unit;
      wWP[lane * 2 * GW + GW + g] = -(wq_r[g] * R.eb_s + wq_i[g] * R.eb_c) * inv_unit;
    }
  }
  load_kmeta(R, c, bh, nn, lane, 0);
  wave_lds_sync();
  float ZA[4], ZB[4], WR[GW][4], WI[GW][4];
  h2v AL[2], BE[2];
  auto ld4 = [&](const float* base, float(&dst)[4]) {
    const float4 a = *reinterpret_cast<const float4*>(base + r * 4);
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
  };
  auto ldh4 = [&](const float* base, h2v(&dst)[2]) {
    const uint2 a = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + r * 4);
    dst[0] = __builtin_bit_cast(h2v, a.x);
    dst[1] = __builtin_bit_cast(h2v, a.y);
  };
  ldh4(wAL, AL);
  ldh4(wBE, BE);
  ld4(wZA, ZA);
  ld4(wZB, ZB);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float* wp = wWP + (4 * r + m) * 2 * GW;
#pragma unroll
    for (int g4 = 0; g4 < 2 * GW; g4 += 4) {
      const float4 x = *reinterpret_cast<const float4*>(wp + g4);
      const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int gg = g4 + u;
        if (gg < GW) WR[gg][m] = xv[u];
        else WI[gg - GW][m] = xv[u];
      }
    }
  }

  // ---- scores of all heads: 16 lanes per token, 4 pairs per lane; the per-head lane
  // sums are a reduce-scatter that leaves head h of the token in lanes 4h'..4h'+3
  // (h' = h for 4 heads, lanes 8h..8h+7 for 2 heads)
  constexpr int KS = Sh::NIT / 2;
  const uint8_t* kcur = k_block<D, BK, KB, VB>(c, bh, n);
  const bool lowhalf = (r & 8) == 0, lowq = (r & 4) == 0;
  // two halves of KS iterations: slot `sl` holds iteration sl of the half; in the first
  // half it is refilled with iteration KS + sl of this block, in the second with
  // iteration sl of the next block (fully unrolled, so that every wait for a slot's
  // load is an exact count of the loads issued after it)
  constexpr int LPH = 16 / GW;  // lanes per head after the reduce-scatter
  // per-lane bases; every iteration adds a compile-time offset (folded into the LDS
  // instructions' offset field)
  const float* tab0 = table + ts * Sh::TPITCH + 8 * r;
  float* sc0 = Sc + ts * GW + r / LPH;
#pragma unroll
  for (int it = 0; it < Sh::NIT; ++it) {
    const int hb = it / KS, sl = it % KS;
    const uint8_t* kref = hb ? knext : kcur + KS * (Sh::TPI * Sh::RK);
    const float* tab = tab0 + it * (Sh::TPI * Sh::TPITCH);
    const uint32_t w = R.k[sl][0];
    load_k_slot(R, sl, sl, kref, koff);
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const f2v a01 = cvt_lo(lo), a23 = cvt_hi(lo), b01 = cvt_lo(hi), b23 = cvt_hi(hi);
    const float ca[4] = {a01.x, a01.y, a23.x, a23.y}, cb[4] = {b01.x, b01.y, b23.x, b23.y};
    const float4 t01 = *reinterpret_cast<const float4*>(tab);
    const float4 t23 = *reinterpret_cast<const float4*>(tab + 4);
    const float cs[4] = {t01.x, t01.z, t23.x, t23.z}, sn[4] = {t01.y, t01.w, t23.y, t23.w};
    float s[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) s[g] = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float ka = __builtin_fmaf((float)AL[m >> 1][m & 1], ca[m], ZA[m]);
      const float kbv = __builtin_fmaf((float)BE[m >> 1][m & 1], cb[m], ZB[m]);
      const float tr = __builtin_fmaf(ka, cs[m], -kbv * sn[m]);
      const float ti = __builtin_fmaf(ka, sn[m], kbv * cs[m]);
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        s[g] = __builtin_fmaf(WR[g][m], tr, s[g]);
        s[g] = __builtin_fmaf(WI[g][m], ti, s[g]);
      }
    }
    float v;
    if constexpr (GW == 4) {
      // lanes r and 15 - r: the low half keeps heads 0, 1, the high half heads 2, 3
      float k0 = lowhalf ? s[0] : s[2], k1 = lowhalf ? s[1] : s[3];
      k0 = add_dpp_rm(k0, lowhalf ? s[2] : s[0]);
      k1 = add_dpp_rm(k1, lowhalf ? s[3] : s[1]);
      // lanes r and 7 - r within the half: the low quad keeps the first of the two
      v = add_dpp_hm(lowq ? k0 : k1, lowq ? k1 : k0);
      v = lanes_sum<4>(v);
    } else {
      v = add_dpp_rm(lowhalf ? s[0] : s[1], lowhalf ? s[1] : s[0]);
      v = lanes_sum<8>(v);
    }
    if (r % LPH == 0) sc0[it * (Sh::TPI * GW)] = v;
    // (iterations are left to the scheduler)
  }
  wave_lds_sync();

  // ---- online softmax per head; lane owns tokens lane and lane + 64
  constexpr int TPL = BK / kWave;  // tokens per lane
  float p[TPL][GW];
  float mloc[GW];
#pragma unroll
  for (int g = 0; g < GW; ++g) mloc[g] = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < TPL; ++k) {
    const int t = lane + kWave * k;
    if constexpr (GW == 4) {
      const float4 v = *reinterpret_cast<const float4*>(Sc + t * 4);
      p[k][0] = v.x; p[k][1] = v.y; p[k][2] = v.z; p[k][3] = v.w;
    } else {
      const float2 v = *reinterpret_cast<const float2*>(Sc + t * 2);
      p[k][0] = v.x; p[k][1] = v.y;
    }
    if constexpr (OUTL) {
      // key outliers of token t: code 0 (dequantized to the zero-point) was stored; add
      // the exact term (x - zero) of each CSR entry, rotated, for every head
      const uint32_t vals = C.kv[k];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = (int)((C.kc[k] >> (8 * q)) & 0xffu);
        const float val = h2f((uint16_t)(vals >> (16 * q)));
        const int i = col % HALF;
        const bool a = col < HALF;
        const float dl = val * unit - (a ? wZA[i] : wZB[i]);   // (x - zero) * u
        const float2 cssn = *reinterpret_cast<const float2*>(table + t * Sh::TPITCH + 2 * i);
        const float* wp = wWP + i * 2 * GW;
#pragma unroll
        for (int g = 0; g < GW; ++g) {
          const float wr = wp[g], wi = -wp[GW + g];   // W / u
          const float re = wr * cssn.x - wi * cssn.y, im = wr * cssn.y + wi * cssn.x;
          p[k][g] += a ? dl * re : -dl * im;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GW; ++g) mloc[g] = fmaxf(mloc[g], p[k][g]);
  }
  if constexpr (OUTL)  // the previous block's
#pragma unroll
    for (int g = 0; g < GW; ++g) merge_vcorr<D>(VCR + g * D, st.acc[g], lane);
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    const float mnew = fmaxf(st.m[g], wave_max_uniform(mloc[g]));
    const float alpha = __builtin_amdgcn_exp2f(st.m[g] - mnew);
    st.m[g] = mnew;
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      p[k][g] = __builtin_amdgcn_exp2f(p[k][g] - mnew);
      psum += p[k][g];
    }
    st.lpart[g] = __builtin_fmaf(st.lpart[g], alpha, psum);
#pragma unroll
    for (int q = 0; q < 4; ++q) st.acc[g][q] *= alpha;
    st.zpart[g][0] *= alpha;
    st.zpart[g][1] *= alpha;
  }
  // ---- value weights w = p * scale per [head][group][token], 16-bit fixed point per
  // (head, group); the zero-point part p * zero is summed in fp32
  uint16_t* Wq16 = reinterpret_cast<uint16_t*>(wl + L.wts);                 // [GW][ng][BK]
  uint32_t* PLN = reinterpret_cast<uint32_t*>(wl + L.wts) + GW * ng * BK / 2;  // [GW][ng][64]
  float wmax[GW][2];
  float inv[GW][2];
#pragma unroll
  for (int g = 0; g < GW; ++g) wmax[g][0] = wmax[g][1] = 0.0f;
  float wv[4][GW];
  float vzc[4];  // this block's value zero-points of elements lane + 64 k
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = lane + 64 * k;
    vzc[k] = 0.0f;
#pragma unroll
    for (int g = 0; g < GW; ++g) wv[k][g] = 0.0f;
    if (e < BK * ng) {
      const int grp = e / BK;
      const int kt = (e % BK) / kWave;  // which of the lane's tokens
      const float vs = h2f(R.vs[k]), vz = h2f(R.vz[k]);
      vzc[k] = vz;
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float pp = p[kt][g];
        wv[k][g] = pp * vs;
        if (grp == 0) {
          st.zpart[g][0] = __builtin_fmaf(pp, vz, st.zpart[g][0]);
          wmax[g][0] = fmaxf(wmax[g][0], wv[k][g]);
        } else {
          st.zpart[g][1] = __builtin_fmaf(pp, vz, st.zpart[g][1]);
          wmax[g][1] = fmaxf(wmax[g][1], wv[k][g]);
        }
      }
    }
  }
  load_vmeta(R, c, bh, nn, lane, ng);
  wave_lds_sync();  // the weight area is reused for the quantized weights below
#pragma unroll
  for (int g = 0; g < GW; ++g) {
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      if (grp < ng) {
        const float w = wave_max_uniform(wmax[g][grp]);
        inv[g][grp] = w * (1.0f / 65535.0f);
        wmax[g][grp] = w > 0.0f ? 65535.0f * __builtin_amdgcn_rcpf(w) : 0.0f;  // now the scale
      } else {
        inv[g][grp] = 0.0f;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = lane + 64 * k;
    if (e < BK * ng) {
      const int grp = e / BK, t = e % BK;
#pragma unroll
      for (int g = 0; g < GW; ++g)
        Wq16[(g * ng + grp) * BK + t] = (uint16_t)__builtin_rintf(wv[k][g] * (grp ? wmax[g][1] : wmax[g][0]));
    }
  }
  wave_lds_sync();
  // nibble planes: plane kk of a token group holds nibble kk of each token's weight,
  // token u of the group at bits [4u, 4u+4) (the bit position of its code in a word)
  for (int hg = 0; hg < GW * ng; ++hg) {
    const uint16_t* wg = Wq16 + hg * BK;
    uint32_t plane = 0;
    if constexpr (VB == 4) {
      const int tg = lane >> 2, kk = lane & 3;
      if (tg < BK / 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(wg + 8 * tg);
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) plane |= ((d[u >> 1] >> (16 * (u & 1) + 4 * kk)) & 15u) << (4 * u);
        PLN[hg * 64 + lane] = plane;
      }
    } else {
      const int tg = lane >> 3, par = (lane >> 2) & 1, kk = lane & 3;
      if (tg < BK / 16) {
        const uint4 w0 = *reinterpret_cast<const uint4*>(wg + 16 * tg);
        const uint4 w1 = *reinterpret_cast<const uint4*>(wg + 16 * tg + 8);
        const uint32_t d[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) plane |= ((d[u] >> (16 * par + 4 * kk)) & 15u) << (4 * u);
        PLN[hg * 64 + lane] = plane;
      }
    }
  }
  wave_lds_sync();

  // ---- values, two heads at a time over the value words held in registers
  const int ch0 = (4 * lane) % D;
  const int grp0 = ch0 / G;
#pragma unroll
  for (int g0 = 0; g0 < GW; g0 += 2) {
    uint32_t ia[2][4][4];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int pl = 0; pl < 4; ++pl) ia[gg][k][pl] = 0;
#pragma unroll
    for (int i = 0; i < Sh::NVI; ++i) {
      const int tgi = i * (256 / D) + (4 * lane) / D;
      const uint32_t words[4] = {R.v[i].x, R.v[i].y, R.v[i].z, R.v[i].w};
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const uint32_t* pb = PLN + ((g0 + gg) * ng + grp0) * 64;
        if constexpr (VB == 4) {
          const uint4 pl = *reinterpret_cast<const uint4*>(pb + 4 * tgi);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            ia[gg][k][0] = __builtin_amdgcn_udot8(pl.x, words[k], ia[gg][k][0], false);
            ia[gg][k][1] = __builtin_amdgcn_udot8(pl.y, words[k], ia[gg][k][1], false);
            ia[gg][k][2] = __builtin_amdgcn_udot8(pl.z, words[k], ia[gg][k][2], false);
            ia[gg][k][3] = __builtin_amdgcn_udot8(pl.w, words[k], ia[gg][k][3], false);
          }
        } else {
          const uint4 pe = *reinterpret_cast<const uint4*>(pb + 8 * tgi);
          const uint4 po = *reinterpret_cast<const uint4*>(pb + 8 * tgi + 4);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t ev = words[k] & 0x33333333u, od = (words[k] >> 2) & 0x33333333u;
            ia[gg][k][0] = __builtin_amdgcn_udot8(pe.x, ev, ia[gg][k][0], false);
            ia[gg][k][1] = __builtin_amdgcn_udot8(pe.y, ev, ia[gg][k][1], false);
            ia[gg][k][2] = __builtin_amdgcn_udot8(pe.z, ev, ia[gg][k][2], false);
            ia[gg][k][3] = __builtin_amdgcn_udot8(pe.w, ev, ia[gg][k][3], false);
            ia[gg][k][0] = __builtin_amdgcn_udot8(po.x, od, ia[gg][k][0], false);
            ia[gg][k][1] = __builtin_amdgcn_udot8(po.y, od, ia[gg][k][1], false);
            ia[gg][k][2] = __builtin_amdgcn_udot8(po.z, od, ia[gg][k][2], false);
            ia[gg][k][3] = __builtin_amdgcn_udot8(po.w, od, ia[gg][k][3], false);
          }
        }
      }
    }
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const float sc = grp0 == 0 ? inv[g0 + gg][0] : inv[g0 + gg][1];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t tot = ia[gg][k][0] + (ia[gg][k][1] << 4) + (ia[gg][k][2] << 8) + (ia[gg][k][3] << 12);
        st.acc[g0 + gg][k] = __builtin_fmaf((float)tot, sc, st.acc[g0 + gg][k]);
      }
    }
  }
  // ---- value outliers: p * (x - zero) scattered into the per-head channel array
  if constexpr (OUTL) {
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const uint32_t vals = C.vv[k];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = (int)((C.vc[k] >> (8 * q)) & 0xffu);
        const int grp = col / G;
        const float dl = h2f((uint16_t)(vals >> (16 * q))) - (grp ? vzc[2 + k] : vzc[k]);
#pragma unroll
        for (int g = 0; g < GW; ++g) atomicAdd(VCR + g * D + col, p[k][g] * dl);
      }
    }
    load_csr_tok<BK, KO>(C, c, bh, nn, lane);
    // merged into the accumulators at the next block's softmax (or the item's end), so
    // that the atomics complete in the shadow of the next block's scores
  }
#pragma unroll
  for (int i = 0; i < Sh::NVI; ++i) load_v(R, i, vnext, lane);
  wave_lds_sync();
}

// Item = (b, kv-head, head set, split): the wave serves GW query heads of the group.
template <int D, int BK, int KB, int VB, int GW, int KO>
__global__ __launch_bounds__(kGqaWaves * 64) void decode_gqa_kernel(kvq_cache c, const uint16_t* __restrict__ q,
                                                                   int64_t q_pos, float* __restrict__ ws, int S,
                                                                   int64_t nitems) {
  using Sh = GShape<D, BK, KB, VB>;
  constexpr int kNT = kGqaWaves * 64;
  extern __shared__ float lds[];
  const int H = c.cfg.kv_heads, Hq = c.cfg.q_heads, gq = Hq / H, nsets = gq / GW;
  const int G = c.cfg.v_group, ng = D / G;
  constexpr bool OUTL = KO > 0;
  const int64_t nfull = c.length / BK;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ts = lane / Sh::LPT, r = lane % Sh::LPT;
  const uint32_t koff = (uint32_t)(ts * Sh::RK + r * (Sh::KW * 4));

  float* table = lds;
  for (int idx = threadIdx.x; idx < BK * Sh::HALF; idx += kNT) {
    const int j = idx / Sh::HALF, i = idx % Sh::HALF;
    *reinterpret_cast<float2*>(table + j * Sh::TPITCH + 2 * i) = *reinterpret_cast<const float2*>(c.rope + 2 * idx);
  }
  const GLds L = gqa_lds(D, BK, GW, ng, OUTL);
  float* wl = lds + BK * Sh::TPITCH + wave * L.total;
  if (OUTL)
    for (int k = lane; k < GW * D; k += kWave) wl[L.vcorr + k] = 0.0f;
  __syncthreads();

  const float unit = cvt_lo(1u).x;  // fp8 value of the byte 1, a power of two
  const float inv_unit = 1.0f / unit;
  const int64_t total_waves = (int64_t)gridDim.x * kGqaWaves;
  for (int64_t item = (int64_t)blockIdx.x * kGqaWaves + wave; item < nitems; item += total_waves) {
    const int split = (int)(item % S);
    const int64_t rest = item / S;
    const int set = (int)(rest % nsets);
    const int64_t bh = rest / nsets;
    const int h = (int)(bh % H);
    const int b = (int)(bh / H);
    const int64_t n0 = nfull * split / S, n1 = nfull * (split + 1) / S;

    // query weights of pair `lane` for each head: scale * conj(q_i) e^{-i f_i q_pos} (fp64)
    float wq_r[GW], wq_i[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) { wq_r[g] = 0.0f; wq_i[g] = 0.0f; }
    if (lane < Sh::HALF) {
      const double f = pow((double)c.cfg.rope_theta, -(2.0 * lane) / (double)D);
      double sn, cs;
      sincos((double)q_pos * f, &sn, &cs);
      const double scl = (double)kLog2e / sqrt((double)D);
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const int hq = h * gq + set * GW + g;
        const uint16_t* qv = q + ((int64_t)b * Hq + hq) * D;
        const double qa = (double)h2f(qv[lane]), qb = (double)h2f(qv[lane + Sh::HALF]);
        wq_r[g] = (float)(scl * (qa * cs - qb * sn));
        wq_i[g] = (float)(-scl * (qa * sn + qb * cs));
      }
    }
    GState<GW> st;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      st.m[g] = -__builtin_inff();
      st.lpart[g] = 0.0f;
      st.acc[g][0] = st.acc[g][1] = st.acc[g][2] = st.acc[g][3] = 0.0f;
      st.zpart[g][0] = st.zpart[g][1] = 0.0f;
    }

    GRegs<D, BK, KB, VB> R;
    CsrTok C;
    if (n0 < n1) {
      load_kmeta(R, c, bh, n0, lane, 0);
      load_vmeta(R, c, bh, n0, lane, ng);
      if constexpr (OUTL) load_csr_tok<BK, KO>(C, c, bh, n0, lane);
      const uint8_t* kb0 = k_block<D, BK, KB, VB>(c, bh, n0);
      const uint8_t* vb0 = v_block<D, BK, KB, VB>(c, bh, n0);
#pragma unroll
      for (int it = 0; it < Sh::NIT / 2; ++it) load_k_slot(R, it, it, kb0, koff);
#pragma unroll
      for (int i = 0; i < Sh::NVI; ++i) load_v(R, i, vb0, lane);
    }
    for (int64_t n = n0; n < n1; ++n)
      gqa_block<D, BK, KB, VB, GW, KO>(R, C, st, wl, L, table, wq_r, wq_i, unit, inv_unit, lane, ts, r, G, ng, c, bh,
                                         n, n + 1 < n1, koff);

    if (OUTL) {
      wave_lds_sync();
#pragma unroll
      for (int g = 0; g < GW; ++g) merge_vcorr<D>(wl + L.vcorr + g * D, st.acc[g], lane);  // the item's last block
      wave_lds_sync();
    }
    // ---- finish the item: reduce across lanes and write (m, l, o) of each head's split
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float l = wave_sum(st.lpart[g]);
      const float z0 = wave_sum(st.zpart[g][0]);
      const float z1 = wave_sum(st.zpart[g][1]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        for (int msk = Sh::CHL; msk < kWave; msk <<= 1) st.acc[g][k] += __shfl_xor(st.acc[g][k], msk, kWave);
      const int hq = h * gq + set * GW + g;
      float* dst = ws + (((int64_t)b * Hq + hq) * S + split) * (D + 2);
      if (lane < Sh::CHL) {
        const int ch0 = 4 * lane;
        const float z = (ch0 / G) == 0 ? z0 : z1;
        *reinterpret_cast<float4*>(dst + 2 + ch0) =
            make_float4(st.acc[g][0] + z, st.acc[g][1] + z, st.acc[g][2] + z, st.acc[g][3] + z);
      }
      if (lane == 0) {
        dst[0] = st.m[g];
        dst[1] = l;
      }
    }
  }
}

template <int D, int BK, int KB, int VB, int GW, int KO>
hipError_t launch_gqa_typed(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S, hipStream_t s,
                            int cus) {
  using Sh = GShape<D, BK, KB, VB>;
  const int ng = c.cfg.head_dim / c.cfg.v_group;
  const GLds L = gqa_lds(D, BK, GW, ng, KO > 0);
  const size_t bytes = ((size_t)BK * Sh::TPITCH + (size_t)kGqaWaves * L.total) * sizeof(float);
  if (bytes > 160 * 1024) return hipErrorNotSupported;
  hipError_t e = hipFuncSetAttribute((const void*)decode_gqa_kernel<D, BK, KB, VB, GW, KO>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  const int gq = c.cfg.q_heads / c.cfg.kv_heads;
  const int64_t nitems = (int64_t)c.cfg.batch * c.cfg.kv_heads * (gq / GW) * S;
  int64_t grid = (nitems + kGqaWaves - 1) / kGqaWaves;
  if (grid > cus) grid = cus;
  hipLaunchKernelGGL((decode_gqa_kernel<D, BK, KB, VB, GW, KO>), dim3((unsigned)grid), dim3(kGqaWaves * 64), bytes,
                     s, c, q, q_pos, ws, S, nitems);
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
  if (gq < 2 || gq % 2 || g.k_mode != 0 || g.k_bits != 4 || (ko != 0 && ko != 2) || ng > 2 ||
      g.k_block * ng > 256 || g.head_dim != 128 || g.k_block != 128)
    return hipErrorNotSupported;
  const int KB = g.k_bits, VB = g.v_bits;
#define KVQ_GQA(kb, vb, gw)                                                                        \
  if (KB == kb && VB == vb && (gq % 4 == 0) == (gw == 4))                                          \
    return ko == 2 ? launch_gqa_typed<128, 128, kb, vb, gw, 2>(c, q, q_pos, ws, S, s, cus)         \
                   : launch_gqa_typed<128, 128, kb, vb, gw, 0>(c, q, q_pos, ws, S, s, cus);
  KVQ_GQA(4, 4, 4) KVQ_GQA(4, 2, 4) KVQ_GQA(4, 4, 2) KVQ_GQA(4, 2, 2)
#undef KVQ_GQA
  return hipErrorNotSupported;
}

}  // namespace kvq
