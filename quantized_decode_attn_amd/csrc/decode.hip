// decode.hip -- decode attention computed directly on the packed cache: the generic
// split kernel (any supported configuration, one query or a causal chunk of queries)
// and the kernel that merges the split partials.
//
// Pages cited (title, address):
//   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
//   [UQ]   "大模型长上下文推理优化：4-bit KV Cache量化技术解析与部署实践", mlqm.cn/news/1064729
//   [TQ]   "TurboQuant：突破大模型推理瓶颈的KVCache量化技术解析", mlqm.cn/news/1002276
//
// Keys are stored before RoPE ([KVC3] "Pre-RoPE Key Quantization"), so the rotation
// is applied at read time.  With channel pairs written as complex numbers
// (k_i + i*k_{i+D/2}) the score of token t against the query at position p is
//     s_t = sum_i Re( conj(q_i) e^{-i f_i p} e^{i f_i t} k_i ) / sqrt(D),
// and t = n*Bk + j factors the rotation into a per-block term and a per-offset term.
// Per block and pair the query-side weight W = conj(q) e^{-i f p} e^{i f n Bk} is
// folded with the block's scale and zero-point (uniform keys) so that one token pair
// costs six fused multiply-adds on its two integer codes plus the cos/sin of j*f
// from an LDS table shared by every block, head and sequence.  Nothing is
// dequantized to memory: the dequantize-then-attend fusion the pages ask for
// ([TQ] sections 5.1 and 6.3; [UQ] section 4.2; the custom kernels of [KVC3]
// "Q-Norm 与其他细节").
//
// Work split (split-K flash decoding): a work item is (b, kv-head, row set, split); a
// split is a contiguous range of Bk-token blocks (the last split of a sequence also
// takes the unquantized tail).  A row is one query vector: query head g of the kv head
// and, for a chunk of nq queries, query j, rotated at q_pos + j and seeing the first
// min(q_pos + j + 1, length) tokens (single-query decode: one query per head, the whole
// cache).  Each wave owns whole items and keeps, for every row of its set, the running
// max m, the running sum l and the unnormalised output o (online softmax in base 2).
// Partials (m, l, o) go to the workspace and a second kernel merges the splits of
// every row in a fixed order.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kFinishMaxSplits = 4096;  // split weights staged in LDS (fp32)
constexpr int kFinishFastSplits = 16;   // merged by one thread per channel with no barrier

template <int D, int KB, int KMODE, int VB>
struct Shape {
  static constexpr int HALF = D / 2;                  // rotary pairs
  static constexpr int PPL = KB == 3 ? 16 : 8;        // pairs per lane
  static constexpr int LPT = HALF / PPL;              // lanes per token
  static constexpr int TPI = kWave / LPT;             // tokens per iteration
  static constexpr int KW = 2 * PPL * KB / 32;        // code dwords per lane per token
  static constexpr int TPW = 32 / VB;                 // tokens per value word
  static constexpr int CPL = D / kWave;               // value channels per lane
  static constexpr int TPITCH = D + 4;                // floats per rope-table row
  static constexpr int NW = 12;                       // floats of per-pair weights
};

typedef float f2v __attribute__((ext_vector_type(2)));

struct WaveLds {  // offsets (in floats) of one wave's scratch area
  int wts, wq, p, ps, vs, vz, state, vc, lut, vlut, total;
};

// nvlut: entries of the value codebook (D * 2^v_bits with codebook values, else 0)
__host__ __device__ inline WaveLds wave_lds(int D, int Bk, int rows, int ng, int tpi, int kb, int kmode,
                                             bool ko, int nvlut) {
  WaveLds w;
  int o = 0;
  w.wts = o; o += (D / 2) * 12;
  w.wq = o; o += rows * D;
  w.p = o; o += Bk;
  w.ps = o; o += Bk * ng;
  w.vs = o; o += Bk * ng;
  w.vz = o; o += Bk * ng;
  w.state = o; o += rows * (D + 2 + ng);
  w.vc = o; o += ko ? tpi * D : 0;
  w.lut = o; o += kmode == 1 ? D * (1 << kb) : 0;
  w.vlut = o; o += nvlut;
  w.total = o;
  return w;
}

template <int KB, int KW>
__device__ __forceinline__ uint32_t get_code(const uint32_t (&w)[KW], int k) {
  const int p = k * KB;
  uint32_t v = w[p >> 5] >> (p & 31);
  if ((p & 31) + KB > 32) v |= w[(p >> 5) + 1] << (32 - (p & 31));
  return v & ((1u << KB) - 1u);
}

// The new token of a fused decode step: its keys and values [B][Hkv][D] (fp16, pre-RoPE)
// stand at tail slot jnew.  Every read of that slot in the step's launches takes the
// input; one launch also writes it into the tail for the steps that follow.  jnew < 0:
// no such token (plain decode, or a step whose token completed a block).
struct StepToken {
  const uint16_t* k;
  const uint16_t* v;
  int jnew;
};

// STEP = false: split kernel, partials to the workspace.  STEP = true: the one-launch
// decode step, one workgroup per (b, kv-head) whose kWaves waves take the kWaves splits;
// the partials are merged in LDS, the output written directly (S must equal kWaves) and
// the step's token stored into the tail.
template <int D, int KB, int KMODE, int VB, bool STEP>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(kvq_cache c,
                                                                const uint16_t* __restrict__ q, RowSpec rs,
                                                                float* __restrict__ ws, int S, int64_t nitems,
                                                                StepToken nt, float* __restrict__ out) {
  using Sh = Shape<D, KB, KMODE, VB>;
  extern __shared__ float lds[];
  const int Bk = c.cfg.k_block;
  const int H = c.cfg.kv_heads, Hq = c.cfg.q_heads, GQ = Hq / H, R = GQ * rs.nq;
  const int G = c.cfg.v_group, ng = D / G;
  const int ko = kout_of(c.cfg);
  const int NK = keep_count(c.cfg);  // keys kept in fp16 per block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ts = lane / Sh::LPT, r = lane % Sh::LPT;

  // rotary offset table cos/sin(j * f_i), j < Bk, shared by the whole workgroup
  float* table = lds;
  for (int idx = threadIdx.x; idx < Bk * Sh::HALF; idx += kThreads) {
    const int j = idx / Sh::HALF, i = idx % Sh::HALF;
    table[j * Sh::TPITCH + 2 * i] = c.rope[2 * idx];
    table[j * Sh::TPITCH + 2 * i + 1] = c.rope[2 * idx + 1];
  }
  const bool vcb = c.cfg.v_mode == 1;  // codebook values
  const bool vf8 = c.cfg.v_mode == 2;  // FP8 values
  constexpr int NLV = 1 << VB;
  const WaveLds L = wave_lds(D, Bk, rs.rpi, ng, Sh::TPI, KB, KMODE, ko > 0, vcb ? D * NLV : 0);
  float* wl = lds + Bk * Sh::TPITCH + wave * L.total;
  float* wts = wl + L.wts;
  float* wq = wl + L.wq;
  float* Pl = wl + L.p;
  float* PS = wl + L.ps;
  float* VS = wl + L.vs;
  float* VZ = wl + L.vz;
  float* state = wl + L.state;
  float* VC = wl + L.vc;
  float* lutl = wl + L.lut;
  float* vlutl = wl + L.vlut;
  const float* rope_blk = c.rope + (int64_t)Bk * D;  // [T/Bk][HALF][2]
  __syncthreads();

  const int64_t total_waves = (int64_t)gridDim.x * kWaves;
  for (int64_t item = (int64_t)blockIdx.x * kWaves + wave; item < nitems; item += total_waves) {
    const int split = (int)(item % S);
    const int64_t rest = item / S;
    const int set = (int)(rest % rs.nsets);
    const int64_t bh = rest / rs.nsets;
    const int h = (int)(bh % H);
    const int b = (int)(bh / H);
    const SlotRow sr = slot_row(c, b, h);
    // the sequence's length (its own in a cache with per-sequence lengths), and the
    // position of its first query (q_pos < 0: the newest token)
    const int64_t len_b = seq_len_of(c, b);
    const int64_t nfull = len_b / Bk;
    const int ntail = (int)(len_b - nfull * Bk);
    const int64_t qbase = rs.q_pos < 0 ? len_b - 1 : rs.q_pos;
    const int row0 = set * rs.rpi;
    const int nrows = R - row0 < rs.rpi ? R - row0 : rs.rpi;
    const int64_t n0 = nfull * split / S, n1 = nfull * (split + 1) / S;
    const bool do_tail = split == S - 1 && ntail > 0;
    // the widest view of the set's rows: no later token is visible to any of them
    int64_t vmax = 0;
    for (int g = 0; g < nrows; ++g) {
      const int64_t v = row_visible(rs, (row0 + g) % rs.nq, len_b);
      vmax = v > vmax ? v : vmax;
    }

    // ---- per item: query weights Wq = scale * conj(q) * e^{-i f p} (fp64), state reset
    for (int g = 0; g < nrows; ++g) {
      const int row = row0 + g, qj = row % rs.nq;
      const uint16_t* qv = q + (((int64_t)b * Hq + (int64_t)h * GQ + row / rs.nq) * rs.nq + qj) * D;
      const int64_t pos = qbase + qj;
      for (int i = lane; i < Sh::HALF; i += kWave) {
        const double qa = (double)h2f(qv[i]), qb = (double)h2f(qv[i + Sh::HALF]);
        const double f = pow((double)c.cfg.rope_theta, -(2.0 * i) / (double)D);
        double sn, cs;
        sincos((double)pos * f, &sn, &cs);
        const double sc = (double)kLog2e / sqrt((double)D);
        wq[g * D + 2 * i] = (float)(sc * (qa * cs - qb * sn));
        wq[g * D + 2 * i + 1] = (float)(-sc * (qa * sn + qb * cs));
      }
      float* st = state + g * (D + 2 + ng);
      for (int k = lane; k < D + 2 + ng; k += kWave) st[k] = k == 0 ? -__builtin_inff() : 0.0f;
    }
    if (KMODE == 1) {
      for (int k = lane; k < D * (1 << KB); k += kWave)
        lutl[k] = h2f(c.k_lut[(int64_t)h * D * (1 << KB) + k]);
    }
    if (vcb)
      for (int k = lane; k < D * NLV; k += kWave) vlutl[k] = h2f(c.v_lut[(int64_t)h * D * NLV + k]);
    wave_lds_sync();

    const int64_t nblocks = (n1 - n0) + (do_tail ? 1 : 0);
    for (int64_t bi = 0; bi < nblocks; ++bi) {
      const bool tail = bi == n1 - n0;
      const int64_t n = tail ? nfull : n0 + bi;
      const int64_t tb = n * Bk;                         // absolute first token
      if (tb >= vmax) break;                             // past every row's view (blocks ascend)
      const int ntok = tail ? ntail : Bk;
      const int iters = (ntok + Sh::TPI - 1) / Sh::TPI;
      // the quantized block's slot (slot_of), its codes and value words
      const int64_t gs = tail ? 0 : slot_at<true>(sr, n);
      const uint8_t* kblk = static_cast<const uint8_t*>(c.k_codes) + gs * Bk * (D * KB / 8);
      const uint32_t* vblk = static_cast<const uint32_t*>(c.v_codes) + gs * (Bk / Sh::TPW) * D;
      // the block's keys kept in fp16: one bit per token offset (Bk <= 128), and a kept
      // token's place among them (their rows are stored in ascending token order)
      uint32_t km[4] = {0u, 0u, 0u, 0u};
      if (!tail && NK > 0)
        for (int r2 = 0; r2 < NK; ++r2) {
          const uint32_t jj = c.k_keep_idx[gs * NK + r2];
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) km[q2] |= (jj >> 5) == (uint32_t)q2 ? 1u << (jj & 31u) : 0u;
        }
      auto kept_pos = [&](int j) -> int {
        const int wsel = j >> 5, bit = j & 31;
        int pos = 0;
        uint32_t wd = 0u;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          if (q2 < wsel) pos += __builtin_popcount(km[q2]);
          if (q2 == wsel) wd = km[q2];
        }
        if (!((wd >> bit) & 1u)) return -1;
        return pos + __builtin_popcount(wd & ((1u << bit) - 1u));
      };

      // value metadata of the block (quantized blocks only)
      if (!tail && !vcb && !vf8) {
        for (int k = lane; k < Bk * ng; k += kWave) {
          const int64_t m = gs * Bk * ng + k;
          VS[k] = h2f(c.v_scale[m]);
          VZ[k] = h2f(c.v_zero[m]);
        }
      }

      for (int g = 0; g < nrows; ++g) {
        // tokens of this block the row sees (a causal row may see none or a prefix)
        const int64_t seen = row_visible(rs, (row0 + g) % rs.nq, len_b) - tb;
        if (seen <= 0) continue;
        const int nvis = seen < ntok ? (int)seen : ntok;
        float* st = state + g * (D + 2 + ng);
        // ---- per block and pair: W = Wq * e^{i f n Bk}, folded with the metadata
        for (int i = lane; i < Sh::HALF; i += kWave) {
          const float qr = wq[g * D + 2 * i], qi = wq[g * D + 2 * i + 1];
          const float cb = rope_blk[(n * Sh::HALF + i) * 2], sb = rope_blk[(n * Sh::HALF + i) * 2 + 1];
          const float wr = qr * cb - qi * sb, wi = qr * sb + qi * cb;
          float* o = wts + i * Sh::NW;
          if (KMODE == 0 && !tail) {
            const int64_t m = gs * D;
            const float al = h2f(c.k_scale[m + i]), be = h2f(c.k_scale[m + i + Sh::HALF]);
            const float za = h2f(c.k_zero[m + i]), zb = h2f(c.k_zero[m + i + Sh::HALF]);
            o[0] = wr * al;
            o[1] = -wi * be;
            o[2] = wr * za - wi * zb;
            o[3] = -wi * al;
            o[4] = -wr * be;
            o[5] = -(wi * za + wr * zb);
            o[6] = za;
            o[7] = zb;
          }
          o[8] = wr;
          o[9] = wi;
        }
        wave_lds_sync();

        // ---- scores: lane (ts, r) covers pairs [r*PPL, r*PPL+PPL) of token it*TPI+ts
        float A1[Sh::PPL], B1[Sh::PPL], Z1[Sh::PPL], A2[Sh::PPL], B2[Sh::PPL], Z2[Sh::PPL];
        float WR[Sh::PPL], WI[Sh::PPL];
#pragma unroll
        for (int m = 0; m < Sh::PPL; ++m) {
          const float* o = wts + (r * Sh::PPL + m) * Sh::NW;
          A1[m] = o[0]; B1[m] = o[1]; Z1[m] = o[2]; A2[m] = o[3]; B2[m] = o[4]; Z2[m] = o[5];
          WR[m] = o[8]; WI[m] = o[9];
        }
        constexpr int MAXIT = 128 / Sh::TPI;  // k_block <= 128
        float sc[MAXIT];
        float mloc = -__builtin_inff();
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
          if (it >= iters) break;
          const int j = it * Sh::TPI + ts;
          float s = 0.0f;
          if (j < ntok) {
            const float* tab = table + j * Sh::TPITCH + 2 * r * Sh::PPL;
            const int kp = tail || NK == 0 ? -1 : kept_pos(j);
            if (!tail && kp < 0) {
              uint32_t w[Sh::KW];
              const uint32_t* src = reinterpret_cast<const uint32_t*>(
                  kblk + j * (D * KB / 8) + r * (Sh::KW * 4));
#pragma unroll
              for (int k = 0; k < Sh::KW; ++k) w[k] = src[k];
#pragma unroll
              for (int m = 0; m < Sh::PPL; ++m) {
                const float cs = tab[2 * m], sn = tab[2 * m + 1];
                const uint32_t ca = get_code<KB, Sh::KW>(w, 2 * m), cb = get_code<KB, Sh::KW>(w, 2 * m + 1);
                float X, Y;
                if (KMODE == 0) {
                  X = __builtin_fmaf(B1[m], (float)cb, __builtin_fmaf(A1[m], (float)ca, Z1[m]));
                  Y = __builtin_fmaf(B2[m], (float)cb, __builtin_fmaf(A2[m], (float)ca, Z2[m]));
                } else {
                  // codebook keys: the channel's entries; FP8 keys: the pair's two bytes
                  // (adjacent in the row) converted together, the hardware conversion
                  // reading OCP E4M3
                  const int ch = r * Sh::PPL + m;
                  float a, bb;
                  if constexpr (KMODE == 2) {
                    const f2v ab = (m & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(w[m >> 1], true)
                                           : __builtin_amdgcn_cvt_pk_f32_fp8(w[m >> 1], false);
                    a = ab.x;
                    bb = ab.y;
                  } else {
                    a = lutl[ch * (1 << KB) + ca];
                    bb = lutl[(ch + Sh::HALF) * (1 << KB) + cb];
                  }
                  X = __builtin_fmaf(WR[m], a, -WI[m] * bb);
                  Y = -__builtin_fmaf(WI[m], a, WR[m] * bb);
                }
                s = __builtin_fmaf(cs, X, __builtin_fmaf(sn, Y, s));
              }
              // outlier corrections: code 0 was stored there, the CSR holds the value
              if (r < ko) {
                const int64_t e = (gs * Bk + j) * ko + r;
                const int col = c.k_col[e];
                const float xo = h2f(c.k_val[e]);
                const int i = col % Sh::HALF;
                const float* o = wts + i * Sh::NW;
                const float cs = table[j * Sh::TPITCH + 2 * i], sn = table[j * Sh::TPITCH + 2 * i + 1];
                const float wr = o[8], wi = o[9];
                float x0;
                if (KMODE == 0) x0 = col < Sh::HALF ? o[6] : o[7];
                else x0 = lutl[col * (1 << KB)];
                const float dlt = xo - x0;
                s += col < Sh::HALF ? dlt * (wr * cs - wi * sn) : -dlt * (wi * cs + wr * sn);
              }
            } else {
              // an fp16 key: a kept key of a quantized block, or a tail token (the step's
              // new token read from the input)
              const uint16_t* kr = !tail ? c.k_keep_val + (gs * NK + kp) * D
                                         : (j == nt.jnew ? nt.k + bh * D : c.k_tail + (bh * Bk + j) * D);
#pragma unroll
              for (int m = 0; m < Sh::PPL; ++m) {
                const int i = r * Sh::PPL + m;
                const float a = h2f(kr[i]), bb = h2f(kr[i + Sh::HALF]);
                const float cs = tab[2 * m], sn = tab[2 * m + 1];
                const float X = __builtin_fmaf(WR[m], a, -WI[m] * bb);
                const float Y = -__builtin_fmaf(WI[m], a, WR[m] * bb);
                s = __builtin_fmaf(cs, X, __builtin_fmaf(sn, Y, s));
              }
            }
          }
          s = group_sum<Sh::LPT>(s);
          if (j >= nvis) s = -__builtin_inff();
          sc[it] = s;
          mloc = fmaxf(mloc, s);
        }
        // ---- online softmax (base 2)
        const float mblk = wave_max(mloc);
        const float mold = st[0];
        const float mnew = fmaxf(mold, mblk);
        const float alpha = exp2f(mold - mnew);
        float lsum = 0.0f;
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
          if (it >= iters) break;
          const int j = it * Sh::TPI + ts;
          const float p = j < nvis ? exp2f(sc[it] - mnew) : 0.0f;
          if (r == 0) {
            lsum += p;
            if (j < ntok) Pl[j] = p;  // 0 for the tokens the row does not see
          }
        }
        lsum = wave_sum(lsum);
        wave_lds_sync();

        // ---- values
        float acc[Sh::CPL];
#pragma unroll
        for (int k = 0; k < Sh::CPL; ++k) acc[k] = st[2 + lane + k * kWave] * alpha;
        if (!tail && vf8) {
          // FP8 values (8-bit value words only): each code is an E4M3 value
          if constexpr (VB == 8)
          for (int gw = 0; gw < Bk / Sh::TPW; ++gw) {
#pragma unroll
            for (int k = 0; k < Sh::CPL; ++k) {
              const uint32_t word = vblk[gw * D + lane + k * kWave];  // 4 tokens' bytes
              const f2v v01 = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
              const f2v v23 = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
              const float vv[4] = {v01.x, v01.y, v23.x, v23.y};
#pragma unroll
              for (int u = 0; u < 4; ++u) acc[k] = __builtin_fmaf(Pl[gw * 4 + u], vv[u], acc[k]);
            }
          }
          if (lane == 0)
            for (int gg = 0; gg < ng; ++gg) st[2 + D + gg] *= alpha;
        } else if (!tail && vcb) {
          // codebook values: each code reads its channel's entry
          for (int gw = 0; gw < Bk / Sh::TPW; ++gw) {
#pragma unroll
            for (int k = 0; k < Sh::CPL; ++k) {
              const int ch = lane + k * kWave;
              const uint32_t word = vblk[gw * D + ch];
              const float* cb = vlutl + ch * NLV;
#pragma unroll
              for (int u = 0; u < Sh::TPW; ++u)
                acc[k] = __builtin_fmaf(Pl[gw * Sh::TPW + u], cb[(word >> (u * VB)) & (NLV - 1u)], acc[k]);
            }
          }
          if (lane == 0)
            for (int gg = 0; gg < ng; ++gg) st[2 + D + gg] *= alpha;
        } else if (!tail) {
          for (int k = lane; k < Bk * ng; k += kWave) PS[k] = Pl[k / ng] * VS[k];
          float zp[8];
          for (int gg = 0; gg < ng; ++gg) zp[gg] = 0.0f;
          for (int t = lane; t < Bk; t += kWave)
            for (int gg = 0; gg < ng; ++gg) zp[gg] = __builtin_fmaf(Pl[t], VZ[t * ng + gg], zp[gg]);
          for (int gg = 0; gg < ng; ++gg) {
            const float z = wave_sum(zp[gg]);
            if (lane == 0) st[2 + D + gg] = st[2 + D + gg] * alpha + z;
          }
          wave_lds_sync();
          for (int gw = 0; gw < Bk / Sh::TPW; ++gw) {
#pragma unroll
            for (int k = 0; k < Sh::CPL; ++k) {
              const int ch = lane + k * kWave;
              const uint32_t word = vblk[gw * D + ch];
              const int grp = ch / G;
#pragma unroll
              for (int u = 0; u < Sh::TPW; ++u) {
                const uint32_t code = (word >> (u * VB)) & ((1u << VB) - 1u);
                acc[k] = __builtin_fmaf(PS[(gw * Sh::TPW + u) * ng + grp], (float)code, acc[k]);
              }
            }
          }
          // value outliers: rows of VC are token slots, so one instruction never
          // updates one address twice
          if (ko > 0) {
            for (int k = lane; k < Sh::TPI * D; k += kWave) VC[k] = 0.0f;
            wave_lds_sync();
            for (int it = 0; it < iters; ++it) {
              const int j = it * Sh::TPI + ts;
              if (r < ko) {
                const int64_t e = (gs * Bk + j) * ko + r;
                const int col = c.v_col[e];
                const float dlt = h2f(c.v_val[e]) - VZ[j * ng + col / G];
                VC[ts * D + col] += Pl[j] * dlt;
              }
              wave_lds_sync();
            }
#pragma unroll
            for (int k = 0; k < Sh::CPL; ++k)
              for (int row = 0; row < Sh::TPI; ++row) acc[k] += VC[row * D + lane + k * kWave];
          }
        } else {
          // fp16 tail values, 16 tokens' loads in flight ahead of their FMAs
          const uint16_t* vt = c.v_tail + bh * Bk * D + lane;
          const uint16_t* vn = nt.v + bh * D + lane;
          int j = 0;
          for (; j + 16 <= nvis; j += 16) {
            uint16_t t[16][Sh::CPL];
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
              for (int k = 0; k < Sh::CPL; ++k)
                t[u][k] = j + u == nt.jnew ? vn[k * kWave] : vt[(int64_t)(j + u) * D + k * kWave];
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
              for (int k = 0; k < Sh::CPL; ++k) acc[k] = __builtin_fmaf(Pl[j + u], h2f(t[u][k]), acc[k]);
          }
          for (; j < nvis; ++j)
#pragma unroll
            for (int k = 0; k < Sh::CPL; ++k)
              acc[k] = __builtin_fmaf(Pl[j], h2f(j == nt.jnew ? vn[k * kWave] : vt[(int64_t)j * D + k * kWave]),
                                      acc[k]);
          if (lane == 0)
            for (int gg = 0; gg < ng; ++gg) st[2 + D + gg] *= alpha;
        }
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < Sh::CPL; ++k) st[2 + lane + k * kWave] = acc[k];
        if (lane == 0) {
          st[0] = mnew;
          st[1] = st[1] * alpha + lsum;
        }
        wave_lds_sync();
      }
    }

    if constexpr (STEP) {
      // the new token into the fp16 tail, for the steps that follow (this launch reads it
      // from the input)
      if (wave == 0 && nt.jnew >= 0)
        for (int k = lane; k < D; k += kWave) {
          c.k_tail[(bh * Bk + nt.jnew) * D + k] = nt.k[bh * D + k];
          c.v_tail[(bh * Bk + nt.jnew) * D + k] = nt.v[bh * D + k];
        }
      break;  // one item per wave: the workgroup's waves hold the kWaves splits of one unit
    }
    // ---- write the partial of every row of the set
    for (int g = 0; g < nrows; ++g) {
      const int row = row0 + g;
      const float* st = state + g * (D + 2 + ng);
      float* dst = ws + ((((int64_t)b * Hq + (int64_t)h * GQ + row / rs.nq) * rs.nq + row % rs.nq) * S + split) *
                            (D + 2);
      for (int k = lane; k < D; k += kWave) dst[2 + k] = st[2 + k] + st[2 + D + k / G];
      if (lane == 0) {
        dst[0] = st[0];
        dst[1] = st[1];
      }
    }
    wave_lds_sync();
  }
  if constexpr (STEP) {
    // ---- merge the waves' (m, l, o) of every row in wave order:
    //   M = max m_w,  out = sum_w o_w 2^(m_w - M) / sum_w l_w 2^(m_w - M)
    __syncthreads();
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const float* st0 = lds + Bk * Sh::TPITCH + L.state;
    for (int idx = threadIdx.x; idx < R * D; idx += kThreads) {
      const int g = idx / D, k = idx % D;
      float M = -__builtin_inff();
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st0[w * L.total + g * (D + 2 + ng)]);
      float Ls = 0.0f, O = 0.0f;
      for (int w = 0; w < kWaves; ++w) {
        const float* st = st0 + w * L.total + g * (D + 2 + ng);
        const float wt = st[0] == -__builtin_inff() ? 0.0f : exp2f(st[0] - M);  // a wave without blocks: 0
        Ls = __builtin_fmaf(st[1], wt, Ls);
        O = __builtin_fmaf(st[2 + k] + st[2 + D + k / G], wt, O);
      }
      out[((int64_t)b * Hq + (int64_t)h * GQ + g) * D + k] = O / Ls;
    }
  }
}

// Finish one row (b, q-head, query j): optionally attend over the unquantized tail
// tokens the row sees (exact fp16 keys and values, the newest length % k_block tokens),
// then merge the S split partials and the tail in a fixed order:
//   M = max m_s,  out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// In a decode step (nt.jnew >= 0) the tail slot jnew is read from the step's token, and
// the first row of every kv head stores that token into the tail.
__global__ __launch_bounds__(256) void decode_finish_kernel(kvq_cache c, const uint16_t* __restrict__ q,
                                                          RowSpec rs, const float* __restrict__ ws,
                                                          float* __restrict__ out, int S, int with_tail,
                                                          StepToken nt) {
  const int D = c.cfg.head_dim, half = D / 2, Bk = c.cfg.k_block;
  const int H = c.cfg.kv_heads, Hq = c.cfg.q_heads, gq = Hq / H;
  const int64_t bq = blockIdx.x;  // row index over [B][Hq][nq]
  const int qj = (int)(bq % rs.nq);
  const int64_t bhq = bq / rs.nq;
  const int b = (int)(bhq / Hq), hq = (int)(bhq % Hq), h = hq / gq;
  const int64_t bh = (int64_t)b * H + h;
  const int64_t len_b = seq_len_of(c, b);
  const int64_t q_pos = (rs.q_pos < 0 ? len_b - 1 : rs.q_pos) + qj;
  const int64_t nfull = len_b / Bk;
  int ntail = with_tail ? (int)(len_b - nfull * Bk) : 0;
  if (ntail > 0) {  // the tail tokens this row sees
    const int64_t seen = row_visible(rs, qj, len_b) - nfull * Bk;
    ntail = seen <= 0 ? 0 : (seen < ntail ? (int)seen : ntail);
  }
  const int tid = threadIdx.x;
  if (nt.jnew >= 0 && hq % gq == 0 && qj == 0 && tid < D) {
    c.k_tail[(bh * Bk + nt.jnew) * D + tid] = nt.k[bh * D + tid];
    c.v_tail[(bh * Bk + nt.jnew) * D + tid] = nt.v[bh * D + tid];
  }
  if (ntail == 0 && S <= kFinishFastSplits) {
    // No tail and few splits: each channel's thread loads every split's (m, l) and its
    // own partial output at once (one memory round trip, no barriers) and merges them
    // in split order:  M = max m_s,  out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
    if (tid >= D) return;
    const float* base = ws + bq * (int64_t)S * (D + 2);
    float mv[kFinishFastSplits], lv[kFinishFastSplits], ov[kFinishFastSplits];
#pragma unroll
    for (int sp = 0; sp < kFinishFastSplits; ++sp) {
      if (sp < S) {
        const float* pp = base + (int64_t)sp * (D + 2);
        mv[sp] = pp[0];
        lv[sp] = pp[1];
        ov[sp] = pp[2 + tid];
      }
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int sp = 0; sp < kFinishFastSplits; ++sp)
      if (sp < S) M = fmaxf(M, mv[sp]);
    float Lsum = 0.0f, O = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kFinishFastSplits; ++sp) {
      if (sp < S) {
        const float w = mv[sp] == -__builtin_inff() ? 0.0f : exp2f(mv[sp] - M);  // empty split: 0
        Lsum = __builtin_fmaf(lv[sp], w, Lsum);
        O = __builtin_fmaf(ov[sp], w, O);
      }
    }
    out[bq * D + tid] = O / Lsum;
    return;
  }
  __shared__ float wr_s[128], wi_s[128], p_s[128], red[8];
  __shared__ float tail_m, tail_l;
  if (ntail > 0) {
    if (tid < half) {
      const uint16_t* qv = q + bq * D;
      const double qa = (double)h2f(qv[tid]), qb = (double)h2f(qv[tid + half]);
      const double f = pow((double)c.cfg.rope_theta, -(2.0 * tid) / (double)D);
      double sn, cs;
      sincos((double)q_pos * f, &sn, &cs);
      const double scl = (double)kLog2e / sqrt((double)D);
      const float qr = (float)(scl * (qa * cs - qb * sn)), qi = (float)(-scl * (qa * sn + qb * cs));
      const float* eb = c.rope + (int64_t)Bk * D + (nfull * half + tid) * 2;
      wr_s[tid] = qr * eb[0] - qi * eb[1];
      wi_s[tid] = qr * eb[1] + qi * eb[0];
    }
    __syncthreads();
    float s = -__builtin_inff();
    if (tid < ntail) {
      const uint16_t* kr = tid == nt.jnew ? nt.k + bh * D : c.k_tail + (bh * Bk + tid) * D;
      const float* tab = c.rope + (int64_t)tid * half * 2;
      s = 0.0f;
      for (int i = 0; i < half; ++i) {
        const float a = h2f(kr[i]), bb = h2f(kr[i + half]);
        const float X = __builtin_fmaf(wr_s[i], a, -wi_s[i] * bb);
        const float Y = -__builtin_fmaf(wi_s[i], a, wr_s[i] * bb);
        s = __builtin_fmaf(tab[2 * i], X, __builtin_fmaf(tab[2 * i + 1], Y, s));
      }
    }
    float m = wave_max(s);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float p = tid < ntail ? exp2f(s - m) : 0.0f;
    if (tid < 128) p_s[tid] = p;
    float l = wave_sum(p);
    __syncthreads();
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = l;
    __syncthreads();
    if (tid == 0) {
      tail_m = m;
      tail_l = (red[4] + red[5]) + (red[6] + red[7]);
    }
    __syncthreads();
  }
  // Merge of the splits (and the tail) in a fixed order.  Split weights
  // w_s = 2^(m_s - M) are formed once in LDS; the channels then read their partial
  // outputs with independent loads, the splits divided between the two thread halves
  // and the halves added in a fixed order.
  __shared__ float wsh[kFinishMaxSplits];
  __shared__ float osh[256], osh_t[256];
  __shared__ float red2[8];
  const float* base = ws + bq * (int64_t)S * (D + 2);
  float mloc = ntail > 0 ? tail_m : -__builtin_inff();
  for (int sp = tid; sp < S; sp += blockDim.x) mloc = fmaxf(mloc, base[(int64_t)sp * (D + 2)]);
  mloc = wave_max(mloc);
  if ((tid & 63) == 0) red2[tid >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red2[0], red2[1]), fmaxf(red2[2], red2[3]));
  float lloc = 0.0f;
  for (int sp = tid; sp < S; sp += blockDim.x) {
    const float* pp = base + (int64_t)sp * (D + 2);
    const float w = pp[0] == -__builtin_inff() ? 0.0f : exp2f(pp[0] - M);  // empty split: 0
    wsh[sp] = w;
    lloc = __builtin_fmaf(pp[1], w, lloc);
  }
  lloc = wave_sum(lloc);
  __syncthreads();
  if ((tid & 63) == 0) red2[4 + (tid >> 6)] = lloc;
  __syncthreads();
  float Lsum = (red2[4] + red2[5]) + (red2[6] + red2[7]);
  const float wt = ntail > 0 ? exp2f(tail_m - M) : 0.0f;
  if (ntail > 0) Lsum = __builtin_fmaf(tail_l, wt, Lsum);
  const int d = tid % D, part = tid / D, nparts = blockDim.x / D;
  const int s0 = S * part / nparts, s1 = S * (part + 1) / nparts;
  // eight loads in flight ahead of the fixed-order FMA chain
  float O = 0.0f;
  int sp = s0;
  for (; sp + 8 <= s1; sp += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = base[(int64_t)(sp + u) * (D + 2) + 2 + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) O = __builtin_fmaf(t[u], wsh[sp + u], O);
  }
  for (; sp < s1; ++sp) O = __builtin_fmaf(base[(int64_t)sp * (D + 2) + 2 + d], wsh[sp], O);
  // the tail's values: tokens j = part, part + nparts, ... of each channel, 16 loads in
  // flight ahead of their FMAs
  float ot = 0.0f;
  if (ntail > 0) {
    const uint16_t* vt = c.v_tail + bh * Bk * D + d;
    const uint16_t* vn = nt.v + bh * D + d;
    int j = part;
    for (; j + 15 * nparts < ntail; j += 16 * nparts) {
      uint16_t t[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int jj = j + u * nparts;
        t[u] = jj == nt.jnew ? vn[0] : vt[(int64_t)jj * D];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) ot = __builtin_fmaf(p_s[j + u * nparts], h2f(t[u]), ot);
    }
    for (; j < ntail; j += nparts) ot = __builtin_fmaf(p_s[j], h2f(j == nt.jnew ? vn[0] : vt[(int64_t)j * D]), ot);
  }
  osh[tid] = O;
  osh_t[tid] = ot;
  __syncthreads();
  if (part == 0) {
    for (int pt = 1; pt < nparts; ++pt) O += osh[pt * D + d];
    if (ntail > 0) {
      for (int pt = 1; pt < nparts; ++pt) ot += osh_t[pt * D + d];
      O = __builtin_fmaf(ot, wt, O);
    }
    out[bq * D + d] = O / Lsum;
  }
}

// 16-bit element e of a row held as uint4 words (e a compile-time index after unrolling).
template <int N>
__device__ __forceinline__ uint16_t row_elem(const uint4 (&w)[N], int e) {
  const uint4& v = w[e >> 3];
  const int k = (e >> 1) & 3;
  const uint32_t x = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  return (uint16_t)(x >> ((e & 1) * 16));
}

// The finish of a row whose kv head has an unquantized tail, for at most
// kFinishFastSplits splits: the same arithmetic as decode_finish_kernel, with every
// global load the row needs (the query, each tail token's key row and rotary offsets,
// the tail values, the split partials) issued before the first is used, so that the row
// costs about one memory round trip instead of one per stage.  Thread tid < ntail scores
// tail token tid; thread (d, part) sums the values of channel d over the tokens
// part, part + NP, ...; the partial sums are added in part order.
template <int D>
__global__ __launch_bounds__(256) void decode_finish_tail_kernel(kvq_cache c, const uint16_t* __restrict__ q,
                                                               RowSpec rs, const float* __restrict__ ws,
                                                               float* __restrict__ out, int S, StepToken nt) {
  constexpr int HALF = D / 2, NP = 256 / D, MAXV = 128 / NP;  // k_block <= 128
  const int Bk = c.cfg.k_block;
  const int H = c.cfg.kv_heads, Hq = c.cfg.q_heads, gq = Hq / H;
  const int64_t bq = blockIdx.x;  // row index over [B][Hq][nq]
  const int qj = (int)(bq % rs.nq);
  const int64_t bhq = bq / rs.nq;
  const int b = (int)(bhq / Hq), hq = (int)(bhq % Hq), h = hq / gq;
  const int64_t bh = (int64_t)b * H + h;
  const int64_t len_b = seq_len_of(c, b);
  const int64_t q_pos = (rs.q_pos < 0 ? len_b - 1 : rs.q_pos) + qj;
  const int64_t nfull = len_b / Bk;
  int ntail = (int)(len_b - nfull * Bk);
  {
    const int64_t seen = row_visible(rs, qj, len_b) - nfull * Bk;
    ntail = seen <= 0 ? 0 : (seen < ntail ? (int)seen : ntail);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = tid % D, part = tid / D;
  if (nt.jnew >= 0 && hq % gq == 0 && qj == 0 && tid < D) {
    c.k_tail[(bh * Bk + nt.jnew) * D + tid] = nt.k[bh * D + tid];
    c.v_tail[(bh * Bk + nt.jnew) * D + tid] = nt.v[bh * D + tid];
  }
  __shared__ float wr_s[HALF], wi_s[HALF], p_s[128], red[8], osh_t[256];

  // ---- every load first
  const float* base = ws + bq * (int64_t)S * (D + 2);
  float mv[kFinishFastSplits], lv[kFinishFastSplits], ov[kFinishFastSplits];
#pragma unroll
  for (int sp = 0; sp < kFinishFastSplits; ++sp) {
    mv[sp] = -__builtin_inff();
    lv[sp] = ov[sp] = 0.0f;
    if (sp < S) {
      mv[sp] = base[(int64_t)sp * (D + 2)];
      lv[sp] = base[(int64_t)sp * (D + 2) + 1];
      if (part == 0) ov[sp] = base[(int64_t)sp * (D + 2) + 2 + d];
    }
  }
  double qa = 0.0, qb = 0.0;
  float eb0 = 0.0f, eb1 = 0.0f, pc = 0.0f, ps = 0.0f, po0 = 0.0f, po1 = 0.0f;
  // inside the capacity, e^{i f q_pos} = e^{i f nb Bk} e^{i f jq} from the fp64-built tables
  const bool qtab = q_pos < c.cfg.capacity;
  if (tid < HALF && ntail > 0) {  // (nfull < T / Bk when there is a tail)
    const uint16_t* qv = q + bq * D;
    qa = (double)h2f(qv[tid]);
    qb = (double)h2f(qv[tid + HALF]);
    const float* eb = c.rope + (int64_t)Bk * D + (nfull * HALF + tid) * 2;
    eb0 = eb[0];
    eb1 = eb[1];
    if (qtab) {
      const float* pb = c.rope + (int64_t)Bk * D + ((q_pos / Bk) * HALF + tid) * 2;
      const float* po = c.rope + ((q_pos % Bk) * HALF + tid) * 2;
      pc = pb[0];
      ps = pb[1];
      po0 = po[0];
      po1 = po[1];
    }
  }
  uint4 kraw[D / 8];
  float4 tab[D / 4];
  if (tid < ntail) {
    if (tid == nt.jnew) {
      const uint16_t* src = nt.k + bh * D;
#pragma unroll
      for (int k = 0; k < D / 8; ++k)
        kraw[k] = make_uint4(src[8 * k] | (uint32_t)src[8 * k + 1] << 16, src[8 * k + 2] | (uint32_t)src[8 * k + 3] << 16,
                             src[8 * k + 4] | (uint32_t)src[8 * k + 5] << 16, src[8 * k + 6] | (uint32_t)src[8 * k + 7] << 16);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(c.k_tail + (bh * Bk + tid) * D);
#pragma unroll
      for (int k = 0; k < D / 8; ++k) kraw[k] = src[k];
    }
    const float4* ts = reinterpret_cast<const float4*>(c.rope + (int64_t)tid * HALF * 2);
#pragma unroll
    for (int k = 0; k < D / 4; ++k) tab[k] = ts[k];
  }
  uint16_t vv[MAXV];
#pragma unroll
  for (int u = 0; u < MAXV; ++u) {
    const int j = part + u * NP;
    vv[u] = j < ntail ? (j == nt.jnew ? nt.v[bh * D + d] : c.v_tail[(bh * Bk + j) * D + d]) : (uint16_t)0;
  }

  // ---- query weights: scale * conj(q) e^{-i f q_pos} (fp64 angle), times the tail
  // block's base rotation e^{i f nfull Bk}
  if (tid < HALF && ntail > 0) {
    double sn, cs;
    if (qtab) {
      cs = (double)(pc * po0 - ps * po1);
      sn = (double)(ps * po0 + pc * po1);
    } else {
      const double f = pow((double)c.cfg.rope_theta, -(2.0 * tid) / (double)D);
      sincos((double)q_pos * f, &sn, &cs);
    }
    const double scl = (double)kLog2e / sqrt((double)D);
    const float qr = (float)(scl * (qa * cs - qb * sn)), qi = (float)(-scl * (qa * sn + qb * cs));
    wr_s[tid] = qr * eb0 - qi * eb1;
    wi_s[tid] = qr * eb1 + qi * eb0;
  }
  __syncthreads();
  // ---- tail scores (base 2) and their softmax
  float s = -__builtin_inff();
  if (tid < ntail) {
    s = 0.0f;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const float a = h2f(row_elem(kraw, i)), bb = h2f(row_elem(kraw, i + HALF));
      const float4 t = tab[i >> 1];
      const float cs = (i & 1) ? t.z : t.x, sn = (i & 1) ? t.w : t.y;
      const float X = __builtin_fmaf(wr_s[i], a, -wi_s[i] * bb);
      const float Y = -__builtin_fmaf(wi_s[i], a, wr_s[i] * bb);
      s = __builtin_fmaf(cs, X, __builtin_fmaf(sn, Y, s));
    }
  }
  const float wm = wave_max(s);
  if (lane == 0) red[wave] = wm;
  __syncthreads();
  const float tm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float p = tid < ntail ? exp2f(s - tm) : 0.0f;
  if (tid < 128) p_s[tid] = p;
  const float wl = wave_sum(p);
  if (lane == 0) red[4 + wave] = wl;
  __syncthreads();
  const float tl = (red[4] + red[5]) + (red[6] + red[7]);

  // ---- merge in split order, then the tail:
  //   M = max(m_s, m_tail),  out = (sum_s o_s 2^(m_s - M) + o_tail 2^(m_tail - M)) / (same for l)
  float M = tm;
#pragma unroll
  for (int sp = 0; sp < kFinishFastSplits; ++sp) M = fmaxf(M, mv[sp]);
  float Lsum = 0.0f, O = 0.0f;
#pragma unroll
  for (int sp = 0; sp < kFinishFastSplits; ++sp) {
    const float w = mv[sp] == -__builtin_inff() ? 0.0f : exp2f(mv[sp] - M);  // empty split: 0
    Lsum = __builtin_fmaf(lv[sp], w, Lsum);
    O = __builtin_fmaf(ov[sp], w, O);
  }
  const float wt = ntail > 0 ? exp2f(tm - M) : 0.0f;
  Lsum = __builtin_fmaf(tl, wt, Lsum);
  float ot = 0.0f;
#pragma unroll
  for (int u = 0; u < MAXV; ++u) {
    const int j = part + u * NP;
    if (j < ntail) ot = __builtin_fmaf(p_s[j], h2f(vv[u]), ot);
  }
  osh_t[tid] = ot;
  __syncthreads();
  if (part == 0) {
#pragma unroll
    for (int pt = 1; pt < NP; ++pt) ot += osh_t[pt * D + d];
    O = __builtin_fmaf(ot, wt, O);
    out[bq * D + d] = O / Lsum;
  }
}

// The finish launch of a decode or chunk: the load-ahead kernel where the rows have an
// unquantized tail to attend over and few splits, else the general one.
hipError_t launch_finish(const kvq_cache& c, const uint16_t* q, RowSpec rs, const float* ws, float* out, int S,
                         int with_tail, StepToken nt, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)c.cfg.batch * c.cfg.q_heads * rs.nq));
  // with per-sequence lengths any sequence may have a tail (a row without one merges
  // its splits alone)
  const bool tail = with_tail && (c.seq_lens || c.length % c.cfg.k_block != 0);
  if (tail && S <= kFinishFastSplits && c.cfg.k_block <= 128) {
    if (c.cfg.head_dim == 128)
      hipLaunchKernelGGL(decode_finish_tail_kernel<128>, grid, dim3(256), 0, s, c, q, rs, ws, out, S, nt);
    else
      hipLaunchKernelGGL(decode_finish_tail_kernel<64>, grid, dim3(256), 0, s, c, q, rs, ws, out, S, nt);
  } else {
    hipLaunchKernelGGL(decode_finish_kernel, grid, dim3(256), 0, s, c, q, rs, ws, out, S, with_tail, nt);
  }
  return hipGetLastError();
}

template <int D, int KB, int KMODE, int VB>
hipError_t launch_typed(const kvq_cache& c, const uint16_t* q, RowSpec rs, float* ws, int S, hipStream_t s,
                        int cus, StepToken nt, float* fused_out) {
  using Sh = Shape<D, KB, KMODE, VB>;
  const int R = c.cfg.q_heads / c.cfg.kv_heads * rs.nq, ng = D / c.cfg.v_group;
  // rows per item: up to 8 (all query heads of a kv head for one query), fewer when
  // their state does not fit the LDS
  int rpi = R < 8 ? R : 8;
  size_t bytes = 0;
  for (;; --rpi) {
    if (rpi < 1) return hipErrorInvalidValue;
    const WaveLds L = wave_lds(D, c.cfg.k_block, rpi, ng, Sh::TPI, KB, KMODE, host_kout(c.cfg) > 0,
                               c.cfg.v_mode == 1 ? D << VB : 0);
    bytes = ((size_t)c.cfg.k_block * Sh::TPITCH + (size_t)kWaves * L.total) * sizeof(float);
    if (bytes <= 160 * 1024) break;
  }
  rs.rpi = rpi;
  rs.nsets = (R + rpi - 1) / rpi;
  if (fused_out) {  // one-launch step: every row of a kv head in one workgroup, its waves the splits
    if (rs.nsets != 1) return hipErrorNotSupported;
    hipError_t e = hipFuncSetAttribute((const void*)decode_split_kernel<D, KB, KMODE, VB, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    const int64_t units = (int64_t)c.cfg.batch * c.cfg.kv_heads;
    hipLaunchKernelGGL((decode_split_kernel<D, KB, KMODE, VB, true>), dim3((unsigned)units), dim3(kThreads), bytes,
                       s, c, q, rs, ws, kWaves, units * kWaves, nt, fused_out);
    return hipGetLastError();
  }
  hipError_t e = hipFuncSetAttribute((const void*)decode_split_kernel<D, KB, KMODE, VB, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  const int64_t nitems = (int64_t)c.cfg.batch * c.cfg.kv_heads * rs.nsets * S;
  int64_t grid = (nitems + kWaves - 1) / kWaves;
  const int64_t cap = (int64_t)cus * (bytes <= 80 * 1024 ? 2 : 1);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((decode_split_kernel<D, KB, KMODE, VB, false>), dim3((unsigned)grid), dim3(kThreads), bytes, s,
                     c, q, rs, ws, S, nitems, nt, nullptr);
  return hipGetLastError();
}

template <int D, int KB, int KMODE>
hipError_t launch_vb(const kvq_cache& c, const uint16_t* q, RowSpec rs, float* ws, int S, hipStream_t s, int cus,
                     StepToken nt, float* fused_out) {
  if (c.cfg.v_bits == 4) return launch_typed<D, KB, KMODE, 4>(c, q, rs, ws, S, s, cus, nt, fused_out);
  if (c.cfg.v_bits == 2) return launch_typed<D, KB, KMODE, 2>(c, q, rs, ws, S, s, cus, nt, fused_out);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_d(const kvq_cache& c, const uint16_t* q, RowSpec rs, float* ws, int S, hipStream_t s, int cus,
                    StepToken nt, float* fused_out) {
  const int kb = c.cfg.k_bits, km = c.cfg.k_mode;
  if (km == 0 && kb == 4) return launch_vb<D, 4, 0>(c, q, rs, ws, S, s, cus, nt, fused_out);
  if (km == 0 && kb == 3) return launch_vb<D, 3, 0>(c, q, rs, ws, S, s, cus, nt, fused_out);
  if (km == 0 && kb == 2) return launch_vb<D, 2, 0>(c, q, rs, ws, S, s, cus, nt, fused_out);
  if (km == 1 && kb == 4) return launch_vb<D, 4, 1>(c, q, rs, ws, S, s, cus, nt, fused_out);
  if (km == 1 && kb == 3) return launch_vb<D, 3, 1>(c, q, rs, ws, S, s, cus, nt, fused_out);
  if (km == 1 && kb == 2) return launch_vb<D, 2, 1>(c, q, rs, ws, S, s, cus, nt, fused_out);
  // FP8 keys come with FP8 values
  if (km == 2 && kb == 8 && c.cfg.v_bits == 8)
    return launch_typed<D, 8, 2, 8>(c, q, rs, ws, S, s, cus, nt, fused_out);
  return hipErrorInvalidValue;
}

hipError_t launch_generic(const kvq_cache& c, const uint16_t* q, RowSpec rs, float* ws, int S, hipStream_t s,
                          int cus, StepToken nt = StepToken{nullptr, nullptr, -1},
                          float* fused_out = nullptr) {
  if (c.cfg.head_dim == 128) return launch_d<128>(c, q, rs, ws, S, s, cus, nt, fused_out);
  if (c.cfg.head_dim == 64) return launch_d<64>(c, q, rs, ws, S, s, cus, nt, fused_out);
  return hipErrorInvalidValue;
}

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus;
}

}  // namespace

hipError_t launch_decode_gqa(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S,
                             hipStream_t s, int cus, bool dry = false);
hipError_t launch_decode_mha(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S,
                             hipStream_t s, int cus, bool dry = false);

// Split kernel + finish kernel; `nt` is the token of a decode step (jnew < 0: none).
// The tuned kernels read quantized blocks only, so the token reaches them through the
// finish kernel, which attends over the tail; the generic kernel reads the tail itself.
static hipError_t decode_two_launches(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* out, float* ws,
                               int splits, hipStream_t s, StepToken nt) {
  const int cus = device_cus();
  const RowSpec rs{q_pos, 1, 0, 1, 1};
  hipError_t e = launch_decode_mha(c, q, q_pos, ws, splits, s, cus);
  if (e == hipErrorNotSupported) e = launch_decode_gqa(c, q, q_pos, ws, splits, s, cus);
  int with_tail = 1;  // the tuned kernels leave the unquantized tail to the finish kernel
  if (e == hipErrorNotSupported) {
    with_tail = 0;
    e = launch_generic(c, q, rs, ws, splits, s, cus, nt);
  }
  if (e != hipSuccess) return e;
  return launch_finish(c, q, rs, ws, out, splits, with_tail, nt, s);
}

hipError_t launch_decode(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* out, float* ws,
                         int splits, hipStream_t s) {
  return decode_two_launches(c, q, q_pos, out, ws, splits, s, StepToken{nullptr, nullptr, -1});
}

bool decode_step_prefers_one_launch(const kvq_cache& c) {
  const kvq_config& g = c.cfg;
  const int D = g.head_dim, R = g.q_heads / g.kv_heads;
  const int ppl = g.k_bits == 3 ? 16 : 8, lpt = D / 2 / ppl, tpi = kWave / lpt;
  const WaveLds L = wave_lds(D, g.k_block, R, D / g.v_group, tpi, g.k_bits, g.k_mode, host_kout(g) > 0,
                             g.v_mode == 1 ? D << g.v_bits : 0);
  const size_t bytes = ((size_t)g.k_block * (D + 4) + (size_t)kWaves * L.total) * sizeof(float);
  if (R > 8 || bytes > 160 * 1024) return false;
  // where a tuned split kernel covers the configuration, it and the finish kernel take
  // less time than the one generic launch
  if (launch_decode_mha(c, nullptr, 0, nullptr, 1, nullptr, 1, true) == hipSuccess) return false;
  if (launch_decode_gqa(c, nullptr, 0, nullptr, 1, nullptr, 1, true) == hipSuccess) return false;
  return true;
}

hipError_t launch_decode_step(const kvq_cache& c, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                              int jnew, float* out, float* ws, int splits, hipStream_t s) {
  const StepToken nt{k_new, v_new, jnew};
  if (splits > 0) return decode_two_launches(c, q, c.length - 1, out, ws, splits, s, nt);
  const RowSpec rs{c.length - 1, 1, 0, 1, 1};
  return launch_generic(c, q, rs, nullptr, kWaves, s, device_cus(), nt, out);
}

hipError_t launch_chunk(const kvq_cache& c, const uint16_t* q, int nq, int64_t q_pos, float* out, float* ws,
                        int splits, hipStream_t s) {
  const int cus = device_cus();
  const RowSpec rs{q_pos, nq, 1, 1, 1};
  hipError_t e = launch_chunk_mfma(c, q, rs, ws, splits, s, cus);
  int with_tail = 1;  // the matrix-core kernel leaves the unquantized tail to the finish kernel
  if (e == hipErrorNotSupported) {
    with_tail = 0;
    e = launch_generic(c, q, rs, ws, splits, s, cus);
  }
  if (e != hipSuccess) return e;
  return launch_finish(c, q, rs, ws, out, splits, with_tail, StepToken{nullptr, nullptr, -1}, s);
}

}  // namespace kvq
