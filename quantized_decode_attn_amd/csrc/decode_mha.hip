// decode_mha.hip -- decode attention over 2/3/4-bit key and 2/4-bit value caches with
// one query head per kv head (multi-head attention), tuned for gfx950.
//
// Pages cited (title, address):
//   [KVC3] "【LLM量化技术介绍-3】KV Cache量化技术介绍", developer.horizon.auto/blog/13163
//   [TQ]   "TurboQuant：突破大模型推理瓶颈的KVCache量化技术解析", mlqm.cn/news/1002276
//
// Same arithmetic as the generic decode kernel: the score of token n*Bk+j is
// sum_i Re(W_n,i e^{i f_i j} (k_a + i k_b)_i) over the rotary pairs i, with W_n,i the
// query weight rotated by the block's first position ([KVC3] "Pre-RoPE Key
// Quantization").  Uniform keys ([KVC3] "Per-Channel Key Quantization") fold the
// block's scale and zero-point into W, six FMAs per pair; codebook keys ([KVC3]
// "Non-Uniform KV Cache Quantization") read (k_a, k_b) of a pair from an LDS table
// indexed by the pair's two codes, built once per kv head and shared by the
// workgroup.  Organised for bandwidth:
//  * 8-wave workgroups share one LDS copy of the cos/sin(j f_i) table;
//  * every wave owns whole (b, head, split) items and streams their blocks through
//    one set of registers: each register slot (codes of one token slot, one 16-byte
//    value load, the metadata) is refilled with block n+1 right after its last use
//    in block n, so a whole block of loads stays in flight;
//  * a key token is covered by 8 lanes (4 for head_dim 64), 8 rotary pairs each,
//    coalesced 4- or 8-byte loads; 4-bit codes masked into 16-bit halves are exact fp16
//    subnormals that the FMAs read in place (v_fma_mix_f32), 2-bit codes become floats
//    two at a time with the packed fp8 conversion (a small byte is an exact fp8 value);
//  * scores go to LDS; each lane then owns two tokens (one for 64-token blocks) for
//    the softmax, the outlier corrections ([KVC3] "Per-Vector Dense-and-Sparse
//    Quantization": code 0 is stored at an outlier, the exact value sits in the CSR)
//    and the value weights;
//  * values are stored as words of consecutive tokens of one channel, so a 16-byte
//    load gives each lane 4 channels x (32 / v_bits) tokens; the per-token weights
//    p*scale are quantized per block to 24-bit fixed point and split into six
//    nibble planes, and the value update is v_dot8_u32_u4 on the packed codes
//    (no unpacking, 8 codes per instruction and plane); codebook values instead add
//    p * entry per code from an LDS copy of the head's codebook.
// The pages' fusion advice ([TQ] sections 5.1 and 6.3) is the design: no dequantized
// value is ever written to memory.
#include <math.h>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dcm;

constexpr int kMhaWaves = 8;  // two waves per SIMD

// Blocks each wave of the workgroup has started.  Waves w and w + 4 share a SIMD, and
// when both are ready the older one wins the issue slot: left alone, waves 0-3 finish
// their items about 1.4 times sooner than waves 4-7, and the later waves then run
// without a partner to hide their latency.  A wave that has started fewer blocks than
// its partner runs one priority level higher until it has caught up, so both stream
// to the end together.  (The counts steer the issue order only: every wave still
// computes exactly its own blocks.)
__shared__ int mha_progress[kMhaWaves];
constexpr float kW24Span = 16776960.0f;  // 2^24 - 2^8: full scale of the fixed-point value weights

// Per-wave LDS area, in floats.
struct MLds {
  int wts, s, ps, vcorr, vlut, total;
};
// nvl: entries per channel of the value codebook (codebook values), else 0
__host__ __device__ inline MLds mha_lds(int D, int BK, bool outl, bool lut, bool keep = false, int nvl = 0) {
  MLds m;
  int o = 0;
  // uniform keys: A1 B1 Z1 A2 B2 Z2 [WR WI [ZA ZB]]; codebook keys: WR WI; one array per name
  m.wts = o; o += (lut ? 2 : outl ? 10 : keep ? 8 : 6) * (D / 2);
  m.s = o; o += BK * (D / 16);                // token scores, as every lane of a token holds it;
                                              // then the fixed-point value weights [2][BK] (u32)
  m.ps = o; o += 256;                         // nibble planes of the value weights [2][16][8]
  m.vcorr = o; o += outl ? D + 4 : 0;         // value outlier corrections [D] (int), then the scale shift
  // value codebook [nvl][D] (fp16): codebook values use no nibble planes and have no
  // outliers, so it starts at the planes' area and runs on past it
  m.vlut = m.ps;
  if (nvl && D * nvl / 2 > 256) o += D * nvl / 2 - 256;
  m.total = o;
  return m;
}

struct MState {
  float m, lpart, acc[4], zpart[2];
};

// Codebook keys: the table entry of rotary pair i and pair code pc = c_a | c_b << KB
// (the two codes as they sit side by side in the row) holds the fp16 codebook values
// (k_a, k_b) in its low and high halves; rows of NPC + 1 entries spread the banks.
template <int KB>
struct PairTab {
  static constexpr int NPC = 1 << (2 * KB);
  static constexpr int PITCH = NPC + 1;
};
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 u32x2_a4 __attribute__((aligned(4)));
typedef __attribute__((address_space(3))) const uint32_t lds_u32;

// Process quantized block n held in R; every register slot is refilled right after
// its last use with block n + 1, or with block n again when `more` is clear (the
// loads stay unconditional, so no register has to survive them).
// Key codes of iteration `it` of a block.  3-bit rows give a lane 48 bits at byte
// 6 r: the 8 bytes from the dword boundary below are loaded (dword alignment suffices
// for the load) and shifted into place at use.
template <int D, int BK, int KB, int VB>
__device__ __forceinline__ void load_codes(BlockRegs<D, BK, KB, VB>& R, int it, const uint8_t* kblk, uint32_t koff) {
  using Sh = MShape<D, BK, KB, VB>;
  if constexpr (KB == 3) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4*>(kblk + koff + it * (Sh::TPI * Sh::RK)));
    R.k[it][0] = x.x;
    R.k[it][1] = x.y;
  } else {
    load_k(R, it, kblk, koff);
  }
}

// Block rotation cos/sin(n Bk f_i) of pair `lane` (codebook keys have no block metadata).
template <int D, int BK, int KB, int VB>
__device__ __forceinline__ void load_eb(BlockRegs<D, BK, KB, VB>& R, const kvq_cache& c, int64_t n, int lane) {
  if (lane < D / 2) {
    const float2 eb = reinterpret_cast<const float2*>(c.rope + (int64_t)BK * D + n * D)[lane];
    R.eb_c = eb.x;
    R.eb_s = eb.y;
  }
}

// Block weights of the block whose metadata R holds, one rotary pair per lane, into the
// wave's LDS area: codebook keys WR WI; uniform keys A1 B1 Z1 A2 B2 Z2, then (WR, WI, ZA,
// ZB) per pair with outliers, WR WI with kept fp16 keys (W = query weight rotated by the block's
// first position, folded with scale and zero).
template <int D, int BK, int KB, int VB, int KO, bool LUT, bool KEEP = false>
__device__ __forceinline__ void write_block_weights(const BlockRegs<D, BK, KB, VB>& R, float* wb, float wq_r,
                                                    float wq_i, float inv_unit, int lane) {
  constexpr int HALF = D / 2;
  if (lane >= HALF) return;
  const float wr = wq_r * R.eb_c - wq_i * R.eb_s;
  const float wi = wq_r * R.eb_s + wq_i * R.eb_c;
  if constexpr (LUT) {
    wb[lane] = wr;
    wb[HALF + lane] = wi;
  } else {
    const float al = h2f(R.kmeta[0]), be = h2f(R.kmeta[1]);
    const float za = h2f(R.kmeta[2]), zb = h2f(R.kmeta[3]);
    // code units: 4-bit codes are read as fp16 subnormals (code_a * 2^-24, code_b * 2^-20),
    // 2-bit codes as fp8 values; powers of two, so the products are unchanged
    const float ua = KB == 4 ? 0x1p24f : inv_unit, ub = KB == 4 ? 0x1p20f : inv_unit;
    wb[lane] = wr * al * ua;                       // A1
    wb[HALF + lane] = -wi * be * ub;               // B1
    wb[2 * HALF + lane] = wr * za - wi * zb;       // Z1
    wb[3 * HALF + lane] = -wi * al * ua;           // A2
    wb[4 * HALF + lane] = -wr * be * ub;           // B2
    wb[5 * HALF + lane] = -(wi * za + wr * zb);    // Z2
    if constexpr (KO > 0) {
      // (WR, WI, ZA, ZB) of the pair side by side: one read per outlier correction
      *reinterpret_cast<float4*>(wb + 6 * HALF + 4 * lane) = make_float4(wr, wi, za, zb);
    } else if constexpr (KEEP) {
      wb[6 * HALF + lane] = wr;                    // WR
      wb[7 * HALF + lane] = wi;                    // WI
    }
  }
}

template <int D, int BK, int KB, int VB, int KO, bool LUT, bool PG, bool KEEP, bool VCB>
__device__ __forceinline__ void process_block(BlockRegs<D, BK, KB, VB>& R, CsrTok& C, MState& st,
                                              float* __restrict__ wl, const MLds& L, const float* __restrict__ table,
                                              const uint32_t* __restrict__ ptab, float wq_r, float wq_i,
                                              float inv_unit, int lane, int ts, int r, uint32_t sh, int G, int ng,
                                              const kvq_cache& c, const SlotRow& sr, int64_t n, int nstep, bool more,
                                              uint32_t koff) {
  using Sh = MShape<D, BK, KB, VB>;
  constexpr bool OUTL = KO > 0;
  static_assert(!(LUT && OUTL), "codebook keys with outliers take the generic kernel");
  constexpr int TPL = BK / kWave;  // tokens per lane in the softmax
  const bool behind = behind_partner<kMhaWaves>(mha_progress, lane);  // wave-uniform
  const int64_t nn = more ? n + nstep : n;
  const int64_t g = slot_at<PG>(sr, n), gnn = more ? slot_at<PG>(sr, nn) : g;
  const uint8_t* knext = k_block<D, BK, KB, VB>(c, gnn);
  const uint8_t* vnext = v_block<D, BK, KB, VB>(c, gnn);
  // this block's weights were written during the previous block (or at the item's start)
  float* wA1 = wl + L.wts;
  float* wB1 = wA1 + Sh::HALF;
  float* wZ1 = wB1 + Sh::HALF;
  float* wA2 = wZ1 + Sh::HALF;
  float* wB2 = wA2 + Sh::HALF;
  float* wZ2 = wB2 + Sh::HALF;
  const float* wOut = wZ2 + Sh::HALF;  // outliers: (WR, WI, ZA, ZB) per pair
  float* Sc = wl + L.s;
  float* PS = wl + L.ps;
  int* VCI = reinterpret_cast<int*>(wl + L.vcorr);

  // value scale/zero and outlier entries of this block: needed only after the scores,
  // so they are loaded here rather than a block ahead (the loads then never stay in
  // flight across the block loop, which would make the compiler drain every load
  // before the next block)
  if constexpr (!VCB) load_vmeta(R, c, g, lane, ng);
  if constexpr (OUTL) load_csr_tok<BK, KO>(C, c, g, lane);
  // keys of this block kept in fp16 (at most 16 rows, stored in ascending token order):
  // lane covers rotary pairs 16 (lane & 3) .. +16 of kept row lane >> 2, channels of both
  // halves; loaded here, used right after the score loop.  Lanes past the last row
  // reload it.
  uint4 kpa[2], kpb[2];
  uint32_t kpj = 0;
  const int NK = KEEP ? keep_count(c.cfg) : 0;
  if constexpr (KEEP) {
    const int64_t row = g * NK + min(lane >> 2, NK - 1);
    const uint4* src = reinterpret_cast<const uint4*>(c.k_keep_val + row * D + 16 * (lane & 3));
    kpa[0] = src[0];
    kpa[1] = src[1];
    kpb[0] = src[Sh::HALF / 8];
    kpb[1] = src[Sh::HALF / 8 + 1];
    kpj = c.k_keep_idx[row];
  }

  // ---- the next block's metadata (its weights are written during this block's values)
  if constexpr (LUT) load_eb(R, c, nn, lane);
  else load_kmeta(R, c, gnn, nn, lane, 0);
  wave_lds_sync();
  float A1[8], B1[8], Z1[8], A2[8], B2[8], Z2[8];
  if constexpr (LUT) {
    const int p0 = r * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 a1 = *reinterpret_cast<const float4*>(wA1 + p0 + 4 * h);
      const float4 b1 = *reinterpret_cast<const float4*>(wB1 + p0 + 4 * h);
      A1[4 * h] = a1.x; A1[4 * h + 1] = a1.y; A1[4 * h + 2] = a1.z; A1[4 * h + 3] = a1.w;
      B1[4 * h] = b1.x; B1[4 * h + 1] = b1.y; B1[4 * h + 2] = b1.z; B1[4 * h + 3] = b1.w;
    }
  } else {
    const int p0 = r * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 a1 = *reinterpret_cast<const float4*>(wA1 + p0 + 4 * h);
      const float4 b1 = *reinterpret_cast<const float4*>(wB1 + p0 + 4 * h);
      const float4 z1 = *reinterpret_cast<const float4*>(wZ1 + p0 + 4 * h);
      const float4 a2 = *reinterpret_cast<const float4*>(wA2 + p0 + 4 * h);
      const float4 b2 = *reinterpret_cast<const float4*>(wB2 + p0 + 4 * h);
      const float4 z2 = *reinterpret_cast<const float4*>(wZ2 + p0 + 4 * h);
      A1[4 * h] = a1.x; A1[4 * h + 1] = a1.y; A1[4 * h + 2] = a1.z; A1[4 * h + 3] = a1.w;
      B1[4 * h] = b1.x; B1[4 * h + 1] = b1.y; B1[4 * h + 2] = b1.z; B1[4 * h + 3] = b1.w;
      Z1[4 * h] = z1.x; Z1[4 * h + 1] = z1.y; Z1[4 * h + 2] = z1.z; Z1[4 * h + 3] = z1.w;
      A2[4 * h] = a2.x; A2[4 * h + 1] = a2.y; A2[4 * h + 2] = a2.z; A2[4 * h + 3] = a2.w;
      B2[4 * h] = b2.x; B2[4 * h + 1] = b2.y; B2[4 * h + 2] = b2.z; B2[4 * h + 3] = b2.w;
      Z2[4 * h] = z2.x; Z2[4 * h + 1] = z2.y; Z2[4 * h + 2] = z2.z; Z2[4 * h + 3] = z2.w;
    }
  }

  if (behind) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
  // ---- scores, summed over a token's lanes and written to LDS by its first lane
  // rotary-table rows in registers one iteration ahead, so the LDS latency of the
  // next token's cos/sin overlaps this token's arithmetic
  float4 tq[2][4];
  const float* tab0 = table + ts * Sh::TPITCH + 4 * r;
  auto load_tab = [&](int it, float4(&t)[4]) {
    const float* tab = tab0 + it * (Sh::TPI * Sh::TPITCH);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) t[q4] = *reinterpret_cast<const float4*>(tab + 4 * Sh::LPT * q4);
  };
  load_tab(0, tq[0]);
  static_assert(Sh::NIT % 4 == 0, "token sums are reduced four iterations at a time");
  float sb[4];
#pragma unroll
  for (int it = 0; it < Sh::NIT; ++it) {
    if (it + 1 < Sh::NIT) load_tab(it + 1, tq[(it + 1) & 1]);
    float s = 0.0f;
    if constexpr (LUT) {
      const uint32_t pt_lds = (uint32_t)(uintptr_t)(const lds_u32*)ptab;
      // pair codes of the lane's 8 pairs, then (k_a, k_b) from the table:
      // X = Re(W k), Y = -Im(W k), score += cos * X + sin * Y
      uint32_t pc[8];
      if constexpr (KB == 3) {
        const uint32_t lo = __builtin_amdgcn_alignbit(R.k[it][1], R.k[it][0], sh);
        const uint32_t hi = R.k[it][1] >> sh;
#pragma unroll
        for (int m = 0; m < 5; ++m) pc[m] = __builtin_amdgcn_ubfe(lo, 6 * m, 6);
        pc[5] = __builtin_amdgcn_alignbit(hi, lo, 30) & 63u;
        pc[6] = __builtin_amdgcn_ubfe(hi, 4, 6);
        pc[7] = __builtin_amdgcn_ubfe(hi, 10, 6);
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) pc[m] = __builtin_amdgcn_ubfe(R.k[it][0], 4 * m, 4);
      }
      load_codes(R, it, knext, koff);
      // entry address = lane base + 4 pc (one shift-add; the pair's row is the
      // instruction's constant offset); all eight lookups issue before their use
      uint32_t kab[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t ea;
        asm("v_lshl_add_u32 %0, %1, 2, %2" : "=v"(ea) : "v"(pc[m]), "v"(pt_lds));
        kab[m] = reinterpret_cast<const lds_u32*>(ea)[m * PairTab<KB>::PITCH];
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the lookups ahead of the arithmetic
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 t = tq[it & 1][q4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int m = 2 * q4 + u;
          const float cs = u ? t.z : t.x, sn = u ? t.w : t.y;
          const h2v kv = __builtin_bit_cast(h2v, kab[m]);
          const float ka = (float)kv.x, kb = (float)kv.y;
          // products with a zero addend stay mixed-precision FMAs (fp16 operand read in place)
          const float X = __builtin_fmaf(A1[m], ka, __builtin_fmaf(-B1[m], kb, 0.0f));
          const float Y = __builtin_fmaf(B1[m], ka, __builtin_fmaf(A1[m], kb, 0.0f));
          s = __builtin_fmaf(cs, X, s);
          s = __builtin_fmaf(-sn, Y, s);
        }
      }
    } else {
      float ca[8], cb[8];
      if constexpr (KB == 4) unpack4_f16<Sh::KW>(R.k[it], ca, cb);
      else unpack_pairs<KB, Sh::KW>(R.k[it], ca, cb);
      load_k(R, it, knext, koff);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 t = tq[it & 1][q4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int m = 2 * q4 + u;
          const float cs = u ? t.z : t.x, sn = u ? t.w : t.y;
          float X = __builtin_fmaf(A1[m], ca[m], Z1[m]);
          X = __builtin_fmaf(B1[m], cb[m], X);
          float Y = __builtin_fmaf(A2[m], ca[m], Z2[m]);
          Y = __builtin_fmaf(B2[m], cb[m], Y);
          s = __builtin_fmaf(cs, X, s);
          s = __builtin_fmaf(sn, Y, s);
        }
      }
    }
    sb[it & 3] = s;
    if ((it & 3) == 3) {
      // every lane stores its four token sums (no branch in the loop)
      lanes_sum4<Sh::LPT>(sb);
      *reinterpret_cast<float4*>(Sc + ((it >> 2) * kWave + lane) * 4) = make_float4(sb[0], sb[1], sb[2], sb[3]);
    }
  }
  wave_lds_sync();

  if constexpr (KEEP) {
    // exact scores of the kept keys, in place of the ones their stored code 0 gave:
    // sum_i a_i (wr_i cos - wi_i sin) - b_i (wi_i cos + wr_i sin) at the token's offset
    const float* wWRk = wl + L.wts + 6 * Sh::HALF;
    const float* wWIk = wWRk + Sh::HALF;
    const int i0 = 16 * (lane & 3);
    const float* tj = table + (int)(kpj & (BK - 1)) * Sh::TPITCH;
    const uint32_t* ha = reinterpret_cast<const uint32_t*>(kpa);
    const uint32_t* hb = reinterpret_cast<const uint32_t*>(kpb);
    float s = 0.0f;
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      const float4 wr4 = *reinterpret_cast<const float4*>(wWRk + i0 + 4 * m4);
      const float4 wi4 = *reinterpret_cast<const float4*>(wWIk + i0 + 4 * m4);
      const float wr[4] = {wr4.x, wr4.y, wr4.z, wr4.w}, wi[4] = {wi4.x, wi4.y, wi4.z, wi4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int m = 4 * m4 + u;
        const float2 cssn = *reinterpret_cast<const float2*>(tj + Sh::tab_off(i0 + m));
        const float a = h2f((uint16_t)(ha[m >> 1] >> (16 * (m & 1))));
        const float bb = h2f((uint16_t)(hb[m >> 1] >> (16 * (m & 1))));
        s = __builtin_fmaf(a, __builtin_fmaf(wr[u], cssn.x, -wi[u] * cssn.y), s);
        s = __builtin_fmaf(-bb, __builtin_fmaf(wi[u], cssn.x, wr[u] * cssn.y), s);
      }
    }
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    if ((lane & 3) == 0 && (lane >> 2) < NK) {
      const int t = (int)(kpj & (BK - 1));
      Sc[((t / Sh::TPI) >> 2) * (4 * kWave) + (t % Sh::TPI) * (4 * Sh::LPT) + ((t / Sh::TPI) & 3)] = s;
    }
    wave_lds_sync();
  }

  // the block's serial part (softmax, value weights, planes, value dot products) runs at
  // a raised wave priority, so that its short dependency chains win issue slots over the
  // other wave's score loop; the priority drops back at the next block's score loop
  if (behind) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(1);

  // ---- online softmax in base 2; lane owns tokens lane + 64 k
  float p[TPL];
  float mloc = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < TPL; ++k) {
    const int t = lane + kWave * k;
    // token t = it TPI + ts sits in the copy of lane ts LPT (iteration group it / 4, slot it % 4)
    p[k] = Sc[((t / Sh::TPI) >> 2) * (4 * kWave) + (t % Sh::TPI) * (4 * Sh::LPT) + ((t / Sh::TPI) & 3)];
    if constexpr (OUTL) {
      // key outliers of token t: code 0 (dequantized to the zero-point) was stored; add
      // the exact term (x - zero) of each CSR entry, rotated
#pragma unroll
      for (int q = 0; q < KO; ++q) {
        const int col = (int)((C.kc[k] >> (8 * q)) & 0xffu);
        const float val = h2f((uint16_t)(C.kv[k] >> (16 * q)));
        const int i = col % Sh::HALF;
        const bool a = col < Sh::HALF;
        const float4 w4 = *reinterpret_cast<const float4*>(wOut + 4 * i);
        const float dl = val - (a ? w4.z : w4.w);
        const float2 cssn = *reinterpret_cast<const float2*>(table + t * Sh::TPITCH + Sh::tab_off(i));
        const float wr = w4.x, wi = w4.y;
        p[k] += a ? dl * (wr * cssn.x - wi * cssn.y) : -dl * (wi * cssn.x + wr * cssn.y);
      }
    }
    mloc = fmaxf(mloc, p[k]);
  }
  if constexpr (OUTL) merge_vcorr<D>(VCI, VCI[D], st.acc, lane);  // the previous block's
  {
    const float mnew = fmaxf(st.m, wave_max_uniform(mloc));
    const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
    st.m = mnew;
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      p[k] = __builtin_amdgcn_exp2f(p[k] - mnew);
      psum += p[k];
    }
    st.lpart = __builtin_fmaf(st.lpart, alpha, psum);
#pragma unroll
    for (int k = 0; k < 4; ++k) st.acc[k] *= alpha;
    st.zpart[0] *= alpha;
    st.zpart[1] *= alpha;
  }

  float vzc[4];  // value zero-points of elements lane + 64 k (uniform values)
  if constexpr (VCB) {
    // ---- codebook values: every token's probability to LDS (over the scores), then
    // acc += p_t * codebook[channel][code] for each code of the lane's value words (the
    // head's fp16 codebook sits in the wave's LDS area); no fixed point, no zero-point
    float* PT = Sc;
    wave_lds_sync();  // every lane has read its scores
#pragma unroll
    for (int k = 0; k < TPL; ++k) PT[lane + kWave * k] = p[k];
    wave_lds_sync();
    write_block_weights<D, BK, KB, VB, KO, LUT, KEEP>(R, wl + L.wts, wq_r, wq_i, inv_unit, lane);
    constexpr int NLV = 1 << VB;
    // [NLV][D], read as fp16 so that the products are mixed-precision FMAs
    const _Float16* book = reinterpret_cast<const _Float16*>(wl + L.vlut);
    const int ch0 = (4 * lane) % D;
#pragma unroll
    for (int i = 0; i < Sh::NVI; ++i) {
      const int g = i * (256 / D) + (4 * lane) / D;  // the load's token group
      const uint32_t words[4] = {R.v[i].x, R.v[i].y, R.v[i].z, R.v[i].w};
      float pp[Sh::TPW];
#pragma unroll
      for (int q4 = 0; q4 < Sh::TPW / 4; ++q4) {
        const float4 f = *reinterpret_cast<const float4*>(PT + g * Sh::TPW + 4 * q4);
        pp[4 * q4] = f.x; pp[4 * q4 + 1] = f.y; pp[4 * q4 + 2] = f.z; pp[4 * q4 + 3] = f.w;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const _Float16* cb = book + ch0 + k;
#pragma unroll
        for (int u = 0; u < Sh::TPW; ++u)
          st.acc[k] = __builtin_fmaf(pp[u], (float)cb[((words[k] >> (u * VB)) & (NLV - 1u)) * D], st.acc[k]);
      }
    }
  } else {
    // ---- value weights w_t = p_t * scale_t per [group][token], quantized per block to
    // 24-bit fixed point for the integer dot products: W = rint(w K) with
    // K = (2^24 - 2^8) / (the block's largest weight), so W < 2^24 and each weight is
    // exact up to half a unit (2^-25 of the block maximum) plus the fp32 rounding of w K
    // (2^-24 of w itself).  Summed over a block the first part is at most
    // BK L 2^-25 max(scale) = 2^-25 BK max|v - z|, below the worst case of a plain fp32
    // sum of the BK products (BK 2^-24 of the largest), however small a weight is next to
    // the block maximum.  The zero-point part p_t * zero_t is summed in fp32.  Element
    // lane + 64 k is token (64 k) % BK + lane of group (64 k) / BK, so its probability is
    // p[((64 k) % BK) / 64].
    uint32_t* W32 = reinterpret_cast<uint32_t*>(Sc);                        // [2][BK], over the scores
    uint32_t* PLN = reinterpret_cast<uint32_t*>(PS);                        // [2][16][8] nibble planes
    float wv[4];
    float wmax0 = 0.0f, wmax1 = 0.0f;
  #pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int grp = (kWave * k) / BK, kt = ((kWave * k) % BK) / kWave;
      wv[k] = 0.0f;
      vzc[k] = 0.0f;
      if (kWave * k < BK * ng) {
        const float pp = p[kt];
        wv[k] = pp * h2f(R.vs[k]);
        const float z = h2f(R.vz[k]);
        vzc[k] = z;
        if (grp == 0) {
          st.zpart[0] = __builtin_fmaf(pp, z, st.zpart[0]);
          wmax0 = fmaxf(wmax0, wv[k]);
        } else {
          st.zpart[1] = __builtin_fmaf(pp, z, st.zpart[1]);
          wmax1 = fmaxf(wmax1, wv[k]);
        }
      }
    }
    wmax0 = wave_max_uniform(wmax0);
    if (ng > 1) wmax1 = wave_max_uniform(wmax1);
    // fixed-point scale and its inverse; they need only agree with each other (to fp32
    // rounding).  wmax * K <= (2^24 - 2^8)(1 + 2^-22) stays below 2^24.
    const float kq0 = wmax0 > 0.0f ? kW24Span * __builtin_amdgcn_rcpf(wmax0) : 0.0f;
    const float kq1 = wmax1 > 0.0f ? kW24Span * __builtin_amdgcn_rcpf(wmax1) : 0.0f;
    wave_lds_sync();  // every lane has read its scores before the weights overwrite them
  #pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = lane + 64 * k;
      if (kWave * k < BK * ng) {
        const float kq = (kWave * k) / BK == 0 ? kq0 : kq1;
        W32[e] = (uint32_t)__builtin_rintf(wv[k] * kq);
      }
    }
    wave_lds_sync();
    // nibble planes: plane n of a token group holds nibble n of each token's weight,
    // token u of the group at bits [4u, 4u+4) (the bit position of its code in a word);
    // a lane builds planes kk and kk + 4 of one token group
    for (int grp = 0; grp < ng; ++grp) {
      const uint32_t* wg = W32 + grp * BK;
      uint32_t plo = 0, phi = 0;
      if constexpr (VB == 4) {
        const int tg = lane >> 2, kk = lane & 3;           // 16 groups of 8 tokens
        if (tg < BK / 8) {
          const uint4 w0 = *reinterpret_cast<const uint4*>(wg + 8 * tg);
          const uint4 w1 = *reinterpret_cast<const uint4*>(wg + 8 * tg + 4);
          const uint32_t d[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  #pragma unroll
          for (int u = 0; u < 8; ++u) {
            plo |= __builtin_amdgcn_ubfe(d[u], 4 * kk, 4) << (4 * u);
            phi |= __builtin_amdgcn_ubfe(d[u], 4 * kk + 16, 4) << (4 * u);
          }
          PLN[grp * 128 + 8 * tg + kk] = plo;
          PLN[grp * 128 + 8 * tg + 4 + kk] = phi;
        }
      } else {
        const int tg = lane >> 3, par = (lane >> 2) & 1, kk = lane & 3;   // 8 groups of 16 tokens
        if (tg < BK / 16) {
          uint32_t d[8];
  #pragma unroll
          for (int h = 0; h < 4; ++h) {  // tokens 2u + par of the group
            const uint4 w = *reinterpret_cast<const uint4*>(wg + 16 * tg + 4 * h);
            d[2 * h] = par ? w.y : w.x;
            d[2 * h + 1] = par ? w.w : w.z;
          }
  #pragma unroll
          for (int u = 0; u < 8; ++u) {
            plo |= __builtin_amdgcn_ubfe(d[u], 4 * kk, 4) << (4 * u);
            phi |= __builtin_amdgcn_ubfe(d[u], 4 * kk + 16, 4) << (4 * u);
          }
          PLN[grp * 128 + 16 * tg + 8 * par + kk] = plo;
          PLN[grp * 128 + 16 * tg + 8 * par + 4 + kk] = phi;
        }
      }
    }
    wave_lds_sync();

    // ---- the next block's weights: this block's were last read by its softmax (key
    // outliers); writing them here lets their LDS round trip overlap the value dot products
    write_block_weights<D, BK, KB, VB, KO, LUT, KEEP>(R, wl + L.wts, wq_r, wq_i, inv_unit, lane);

    // ---- values: lane owns channels ch0..ch0+3, the token group changes with the load;
    // sum_t w_t * code_t by 4-bit integer dot products over the six weight nibbles, in
    // two passes (bits 16..23, then 0..15) that share the accumulator registers.  A plane
    // sum is at most BK * 15 * 15 = 28,800, so four planes combine exactly in 32 bits.
    const int ch0 = (4 * lane) % D;
    const int grp0 = ch0 / G;
    const float inv = (grp0 == 0 ? wmax0 : wmax1) * (1.0f / kW24Span);
  #pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int poff = pass == 0 ? 4 : 0;  // plane offset within a token group's eight
      const int npl = pass == 0 ? 2 : 4;   // planes 4 and 5 hold bits 16..23; 6 and 7 are zero
      uint32_t ia[4][4];
  #pragma unroll
      for (int k = 0; k < 4; ++k)
  #pragma unroll
        for (int pl = 0; pl < 4; ++pl) ia[k][pl] = 0;
  #pragma unroll
      for (int i = 0; i < Sh::NVI; ++i) {
        const int g = i * (256 / D) + (4 * lane) / D;
        const uint32_t words[4] = {R.v[i].x, R.v[i].y, R.v[i].z, R.v[i].w};
        if constexpr (VB == 4) {
          const uint4 pl = *reinterpret_cast<const uint4*>(PLN + grp0 * 128 + 8 * g + poff);
  #pragma unroll
          for (int k = 0; k < 4; ++k) {
            ia[k][0] = __builtin_amdgcn_udot8(pl.x, words[k], ia[k][0], false);
            ia[k][1] = __builtin_amdgcn_udot8(pl.y, words[k], ia[k][1], false);
            if (npl == 4) {
              ia[k][2] = __builtin_amdgcn_udot8(pl.z, words[k], ia[k][2], false);
              ia[k][3] = __builtin_amdgcn_udot8(pl.w, words[k], ia[k][3], false);
            }
          }
        } else {
          const uint4 pe = *reinterpret_cast<const uint4*>(PLN + grp0 * 128 + 16 * g + poff);
          const uint4 po = *reinterpret_cast<const uint4*>(PLN + grp0 * 128 + 16 * g + 8 + poff);
  #pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t ev = words[k] & 0x33333333u, od = (words[k] >> 2) & 0x33333333u;
            ia[k][0] = __builtin_amdgcn_udot8(pe.x, ev, ia[k][0], false);
            ia[k][1] = __builtin_amdgcn_udot8(pe.y, ev, ia[k][1], false);
            ia[k][0] = __builtin_amdgcn_udot8(po.x, od, ia[k][0], false);
            ia[k][1] = __builtin_amdgcn_udot8(po.y, od, ia[k][1], false);
            if (npl == 4) {
              ia[k][2] = __builtin_amdgcn_udot8(pe.z, ev, ia[k][2], false);
              ia[k][3] = __builtin_amdgcn_udot8(pe.w, ev, ia[k][3], false);
              ia[k][2] = __builtin_amdgcn_udot8(po.z, od, ia[k][2], false);
              ia[k][3] = __builtin_amdgcn_udot8(po.w, od, ia[k][3], false);
            }
          }
        }
      }
      const float unit = pass == 0 ? inv * 65536.0f : inv;
  #pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t tot = ia[k][0] + (ia[k][1] << 4) + (ia[k][2] << 8) + (ia[k][3] << 12);
        st.acc[k] = __builtin_fmaf((float)tot, unit, st.acc[k]);
      }
    }

  }
  // ---- value outliers: p * (x - zero) scattered into the channel array, merged into
  // the accumulators at the next block's softmax (or the item's end), so that the
  // atomics complete in the shadow of the next block's scores
  if constexpr (OUTL) {
    float cr[TPL][KO];
    int col[TPL][KO];
    float csum = 0.0f;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
#pragma unroll
      for (int q = 0; q < KO; ++q) {
        col[k][q] = (int)((C.vc[k] >> (8 * q)) & 0xffu);
        const float dl = h2f((uint16_t)(C.vv[k] >> (16 * q))) - (col[k][q] >= G ? vzc[TPL + k] : vzc[k]);
        cr[k][q] = p[k] * dl;
        csum += fabsf(cr[k][q]);
      }
    }
    const int vsh = vcorr_shift(wave_sum_uniform(csum));
    if (lane == 0) VCI[D] = vsh;
#pragma unroll
    for (int k = 0; k < TPL; ++k)
#pragma unroll
      for (int q = 0; q < KO; ++q) atomicAdd(VCI + col[k][q], vcorr_fixed(cr[k][q], vsh));
  }
#pragma unroll
  for (int i = 0; i < Sh::NVI; ++i) load_v(R, i, vnext, lane);
  wave_lds_sync();
}

// One (b, head, split) item on one wave: every full block of the split, then the
// split's (m, l, o) to the workspace.
template <int D, int BK, int KB, int VB, int KO, bool LUT, bool PG, bool KEEP, bool VCB>
__device__ __forceinline__ void mha_item(const kvq_cache& c, const uint16_t* __restrict__ q, int64_t q_pos,
                                         float* __restrict__ ws, int S, int64_t bh, int split, float* wl,
                                         const MLds& L, const float* table, const uint32_t* ptab, int lane) {
  using Sh = MShape<D, BK, KB, VB>;
  constexpr bool OUTL = KO > 0;
  const int H = c.cfg.kv_heads;
  const int G = c.cfg.v_group, ng = D / G;
  const int h = (int)(bh % H);
  const int b = (int)(bh / H);
  // the sequence's own length and newest position in a cache with per-sequence lengths
  const int64_t len_b = seq_len_t<PG>(c, b);
  const int64_t nfull = len_b / BK;
  if (q_pos < 0) q_pos = len_b - 1;
  const int ts = lane / Sh::LPT, r = lane % Sh::LPT;
  // 3-bit rows: the lane's 48 bits start at byte 6 r, loaded from the dword below
  const uint32_t koff = KB == 3 ? (uint32_t)(ts * Sh::RK + ((6 * r) & ~3)) : (uint32_t)(ts * Sh::RK + r * (Sh::KW * 4));
  const uint32_t sh = KB == 3 ? (uint32_t)(((6 * r) & 3) * 8) : 0u;
  const uint32_t* pt = LUT ? ptab + r * 8 * PairTab<KB>::PITCH : nullptr;
  const float inv_unit = 1.0f / cvt_lo(1u).x;  // fp8 value of the byte 1
  // split `split` takes blocks split, split + S, split + 2 S, ...: the waves of a
  // workgroup hold consecutive splits of one head, so at any time they stream
  // neighbouring blocks (contiguous runs of HBM rather than S scattered streams)
  const int64_t n0 = split;

  // query weight of pair `lane`: scale * conj(q_i) * e^{-i f_i q_pos}, evaluated in fp64
  float wq_r = 0.0f, wq_i = 0.0f;
  if (lane < Sh::HALF) {
    const uint16_t* qv = q + ((int64_t)b * H + h) * D;
    const double qa = (double)h2f(qv[lane]), qb = (double)h2f(qv[lane + Sh::HALF]);
    const double f = pow((double)c.cfg.rope_theta, -(2.0 * lane) / (double)D);
    double sn, cs;
    sincos((double)q_pos * f, &sn, &cs);
    const double scl = (double)kLog2e / sqrt((double)D);
    wq_r = (float)(scl * (qa * cs - qb * sn));
    wq_i = (float)(-scl * (qa * sn + qb * cs));
  }
  MState st;
  st.m = -__builtin_inff();
  st.lpart = 0.0f;
  st.acc[0] = st.acc[1] = st.acc[2] = st.acc[3] = 0.0f;
  st.zpart[0] = st.zpart[1] = 0.0f;

  BlockRegs<D, BK, KB, VB> R;
  CsrTok C;
  const SlotRow sr = slot_row(c, b, h);
  if constexpr (VCB) {
    // the head's value codebook into the wave's LDS area, code-major ([code][channel]):
    // a wave's lookups then spread over the banks by channel
    constexpr int NLV = 1 << VB;
    const uint16_t* src = c.v_lut + (int64_t)h * D * NLV;  // [channel][code]
    uint16_t* dst = reinterpret_cast<uint16_t*>(wl + L.vlut);
    for (int k = lane; k < D * NLV; k += kWave) dst[(k % NLV) * D + k / NLV] = src[k];
    wave_lds_sync();
  }
  if (n0 < nfull) {
    const int64_t g0 = slot_at<PG>(sr, n0);
    if constexpr (LUT) load_eb(R, c, n0, lane);
    else load_kmeta(R, c, g0, n0, lane, 0);
    write_block_weights<D, BK, KB, VB, KO, LUT, KEEP>(R, wl + L.wts, wq_r, wq_i, inv_unit, lane);
    const uint8_t* kb0 = k_block<D, BK, KB, VB>(c, g0);
    const uint8_t* vb0 = v_block<D, BK, KB, VB>(c, g0);
#pragma unroll
    for (int it = 0; it < Sh::NIT; ++it) load_codes(R, it, kb0, koff);
#pragma unroll
    for (int i = 0; i < Sh::NVI; ++i) load_v(R, i, vb0, lane);
  }
  for (int64_t n = n0; n < nfull; n += S)
    process_block<D, BK, KB, VB, KO, LUT, PG, KEEP, VCB>(R, C, st, wl, L, table, pt, wq_r, wq_i, inv_unit, lane, ts, r, sh, G, ng,
                                          c, sr, n, S, n + S < nfull, koff);
  if (OUTL) {
    wave_lds_sync();
    int* vci = reinterpret_cast<int*>(wl + L.vcorr);
    merge_vcorr<D>(vci, vci[D], st.acc, lane);  // the item's last block
    wave_lds_sync();
  }

  // ---- finish the item: reduce across lanes and write (m, l, o) of this split
  const float l = wave_sum(st.lpart);
  const float z0 = wave_sum(st.zpart[0]);
  const float z1 = wave_sum(st.zpart[1]);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    for (int msk = Sh::CHL; msk < kWave; msk <<= 1) st.acc[k] += __shfl_xor(st.acc[k], msk, kWave);
  float* dst = ws + (bh * S + split) * (D + 2);
  if (lane < Sh::CHL) {
    const int ch0 = 4 * lane;
    const float z = (ch0 / G) == 0 ? z0 : z1;
    *reinterpret_cast<float4*>(dst + 2 + ch0) =
        make_float4(st.acc[0] + z, st.acc[1] + z, st.acc[2] + z, st.acc[3] + z);
  }
  if (lane == 0) {
    dst[0] = st.m;
    dst[1] = l;
  }
}

// Copies the cos/sin(j f_i) table of a block's offsets into LDS (rows of MShape's
// pitch, pair i at MShape::tab_off(i)).
template <int D, int BK, int NT>
__device__ __forceinline__ void stage_rope(float* table, const kvq_cache& c) {
  using Sh = MShape<D, BK, 4, 4>;
  for (int idx = threadIdx.x; idx < BK * Sh::HALF; idx += NT) {
    const int j = idx / Sh::HALF, i = idx % Sh::HALF;
    *reinterpret_cast<float2*>(table + j * Sh::TPITCH + Sh::tab_off(i)) =
        *reinterpret_cast<const float2*>(c.rope + 2 * idx);
  }
}

// Uniform keys: every wave takes items on its own.  PG: per-sequence lengths (dense or
// paged slots); KEEP: keys kept in fp16 by norm.
template <int D, int BK, int KB, int VB, int KO, bool PG, bool KEEP = false, bool VCB = false>
__global__ __launch_bounds__(kMhaWaves * 64) void decode_mha_kernel(kvq_cache c, const uint16_t* __restrict__ q,
                                                                   int64_t q_pos, float* __restrict__ ws, int S,
                                                                   int64_t nitems, const SeqOrder ord) {
  using Sh = MShape<D, BK, KB, VB>;
  constexpr int kNT = kMhaWaves * 64;
  constexpr bool OUTL = KO > 0;
  extern __shared__ float lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave

  float* table = lds;
  stage_rope<D, BK, kNT>(table, c);
  const MLds L = mha_lds(D, BK, OUTL, false, KEEP, VCB ? 1 << VB : 0);
  float* wl = lds + BK * Sh::TPITCH + wave * L.total;
  if (OUTL)
    for (int k = lane; k < D + 4; k += kWave) reinterpret_cast<int*>(wl + L.vcorr)[k] = 0;
  if (threadIdx.x < kMhaWaves) mha_progress[threadIdx.x] = 0;
  __syncthreads();

  const int64_t total_waves = (int64_t)gridDim.x * kMhaWaves;
  const int64_t p = (int64_t)blockIdx.x * kMhaWaves + wave;
  if constexpr (PG) {  // items in length order, dealt in a snake (every wave exits once k passes nitems)
    const int64_t per_seq = (int64_t)c.cfg.kv_heads * S;
    for (int64_t r = 0;; ++r) {
      const int64_t k = snake_item(r, p, total_waves);
      if (k >= nitems) break;
      const int64_t item = ordered_item(ord, k, per_seq);
      mha_item<D, BK, KB, VB, KO, false, PG, KEEP, VCB>(c, q, q_pos, ws, S, item / S, (int)(item % S), wl, L, table,
                                                        nullptr, lane);
    }
  } else {
    for (int64_t item = p; item < nitems; item += total_waves)
      mha_item<D, BK, KB, VB, KO, false, PG, KEEP, VCB>(c, q, q_pos, ws, S, item / S, (int)(item % S), wl, L, table,
                                                        nullptr, lane);
  }
}

// Codebook keys: the workgroup takes groups of up to 8 splits of one (b, head), so
// that its waves share the head's pair table, rebuilt at every group.  PG: per-sequence
// lengths (dense or paged slots).
template <int D, int BK, int KB, int VB, bool PG>
__global__ __launch_bounds__(kMhaWaves * 64) void decode_mha_lut_kernel(kvq_cache c, const uint16_t* __restrict__ q,
                                                                       int64_t q_pos, float* __restrict__ ws, int S,
                                                                       int64_t ngroups) {
  using Sh = MShape<D, BK, KB, VB>;
  using PT = PairTab<KB>;
  constexpr int kNT = kMhaWaves * 64;
  constexpr int NL = 1 << KB;  // codebook entries per channel
  extern __shared__ float lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = c.cfg.kv_heads;

  float* table = lds;
  stage_rope<D, BK, kNT>(table, c);
  uint32_t* ptab = reinterpret_cast<uint32_t*>(lds + BK * Sh::TPITCH);
  const MLds L = mha_lds(D, BK, false, true);
  float* wl = reinterpret_cast<float*>(ptab + Sh::HALF * PT::PITCH) + wave * L.total;

  const int gps = (S + kMhaWaves - 1) / kMhaWaves;  // groups per (b, head)
  if (threadIdx.x < kMhaWaves) mha_progress[threadIdx.x] = 0;  // published by the loop's first barrier
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t bh = g / gps;
    const int split = (int)(g % gps) * kMhaWaves + wave;
    const uint16_t* lut = c.k_lut + (int64_t)(bh % H) * D * NL;  // [D][NL]
    __syncthreads();  // the previous group is done with the table
    for (int idx = threadIdx.x; idx < Sh::HALF * PT::NPC; idx += kNT) {
      const int i = idx / PT::NPC, pc = idx % PT::NPC;
      const uint32_t ka = lut[i * NL + (pc & (NL - 1))];
      const uint32_t kb = lut[(i + Sh::HALF) * NL + (pc >> KB)];
      ptab[i * PT::PITCH + pc] = ka | (kb << 16);
    }
    __syncthreads();
    if (split < S) mha_item<D, BK, KB, VB, 0, true, PG, false, false>(c, q, q_pos, ws, S, bh, split, wl, L, table, ptab, lane);
  }
}

}  // namespace

// Returns hipErrorNotSupported when the configuration is not one this kernel covers; with
// `dry` it launches nothing and only reports whether it does.
hipError_t launch_decode_mha(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S,
                             hipStream_t s, int cus, bool dry);

template <int D, int BK, int KB, int VB, int KO, bool PG = false, bool KEEP = false, bool VCB = false>
static hipError_t launch_mha_typed(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S,
                                   hipStream_t s, int cus, bool dry) {
  using Sh = MShape<D, BK, KB, VB>;
  const MLds L = mha_lds(D, BK, KO > 0, false, KEEP, VCB ? 1 << VB : 0);
  const size_t bytes = ((size_t)BK * Sh::TPITCH + (size_t)kMhaWaves * L.total) * sizeof(float);
  if (bytes + kMhaWaves * sizeof(int) > 160 * 1024) return hipErrorNotSupported;  // with the static progress counts
  if (dry) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)decode_mha_kernel<D, BK, KB, VB, KO, PG, KEEP, VCB>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  const int64_t nitems = (int64_t)c.cfg.batch * c.cfg.kv_heads * S;
  int64_t grid = (nitems + kMhaWaves - 1) / kMhaWaves;
  if (grid > cus) grid = cus;
  hipLaunchKernelGGL((decode_mha_kernel<D, BK, KB, VB, KO, PG, KEEP, VCB>), dim3((unsigned)grid), dim3(kMhaWaves * 64), bytes, s, c,
                     q, q_pos, ws, S, nitems, PG ? seq_order(c) : SeqOrder{0, {}});
  return hipGetLastError();
}

template <int D, int BK, int KB, int VB, bool PG = false>
static hipError_t launch_mha_lut_typed(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S,
                                       hipStream_t s, int cus, bool dry) {
  using Sh = MShape<D, BK, KB, VB>;
  const MLds L = mha_lds(D, BK, false, true);
  const size_t bytes = ((size_t)BK * Sh::TPITCH + (size_t)Sh::HALF * PairTab<KB>::PITCH +
                        (size_t)kMhaWaves * L.total) * sizeof(float);
  if (bytes + kMhaWaves * sizeof(int) > 160 * 1024) return hipErrorNotSupported;  // with the static progress counts
  if (dry) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)decode_mha_lut_kernel<D, BK, KB, VB, PG>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  const int64_t ngroups = (int64_t)c.cfg.batch * c.cfg.kv_heads * ((S + kMhaWaves - 1) / kMhaWaves);
  const int64_t grid = ngroups < cus ? ngroups : cus;
  hipLaunchKernelGGL((decode_mha_lut_kernel<D, BK, KB, VB, PG>), dim3((unsigned)grid), dim3(kMhaWaves * 64), bytes, s,
                     c, q, q_pos, ws, S, ngroups);
  return hipGetLastError();
}

hipError_t launch_decode_mha(const kvq_cache& c, const uint16_t* q, int64_t q_pos, float* ws, int S,
                             hipStream_t s, int cus, bool dry) {
  const kvq_config& g = c.cfg;
  const int ko = host_kout(g);
  const int ng = g.head_dim / g.v_group;
  if (g.q_heads != g.kv_heads || ko > 2 || ng > 2 || g.k_block * ng > 256) return hipErrorNotSupported;
  if (g.v_mode == 2 || g.k_mode == 2) return hipErrorNotSupported;  // FP8: the generic kernel
  if (g.v_mode != 0) {
    // codebook values (no outliers by construction): uniform 4-bit keys at head_dim 128
    // and 128-token blocks, 2- or 4-bit values, dense or per-sequence, no kept keys;
    // everything else takes the generic kernel
    if (g.head_dim != 128 || g.k_block != 128 || g.k_bits != 4 || g.k_mode != 0 || ko != 0 || g.keep_pct > 0)
      return hipErrorNotSupported;
    if (g.v_bits == 4)
      return c.seq_lens ? launch_mha_typed<128, 128, 4, 4, 0, true, false, true>(c, q, q_pos, ws, S, s, cus, dry)
                        : launch_mha_typed<128, 128, 4, 4, 0, false, false, true>(c, q, q_pos, ws, S, s, cus, dry);
    if (g.v_bits == 2)
      return c.seq_lens ? launch_mha_typed<128, 128, 4, 2, 0, true, false, true>(c, q, q_pos, ws, S, s, cus, dry)
                        : launch_mha_typed<128, 128, 4, 2, 0, false, false, true>(c, q, q_pos, ws, S, s, cus, dry);
    return hipErrorNotSupported;
  }
  const int D = g.head_dim, BK = g.k_block, KB = g.k_bits, VB = g.v_bits;
  if (g.keep_pct > 0) {
    // keys kept in fp16 (uniform keys without outliers): 4-bit keys at head_dim 128 and
    // 128-token blocks, dense or per-sequence; every other configuration takes the
    // generic kernel
    if (D != 128 || BK != 128 || KB != 4 || g.k_mode != 0 || ko != 0) return hipErrorNotSupported;
    if (VB == 4)
      return c.seq_lens ? launch_mha_typed<128, 128, 4, 4, 0, true, true>(c, q, q_pos, ws, S, s, cus, dry)
                        : launch_mha_typed<128, 128, 4, 4, 0, false, true>(c, q, q_pos, ws, S, s, cus, dry);
    if (VB == 2)
      return c.seq_lens ? launch_mha_typed<128, 128, 4, 2, 0, true, true>(c, q, q_pos, ws, S, s, cus, dry)
                        : launch_mha_typed<128, 128, 4, 2, 0, false, true>(c, q, q_pos, ws, S, s, cus, dry);
    return hipErrorNotSupported;
  }
  if (c.seq_lens) {
    // per-sequence lengths (dense or paged slots): uniform 4-bit keys and 2/3-bit
    // codebook keys at head_dim 128; every other configuration takes the generic kernel
    if (D != 128) return hipErrorNotSupported;
    if (g.k_mode == 1) {
      if (ko != 0 || (KB != 3 && KB != 2)) return hipErrorNotSupported;
#define KVQ_MHA_LUT_PG(bk, kb, vb) \
  if (BK == bk && KB == kb && VB == vb) return launch_mha_lut_typed<128, bk, kb, vb, true>(c, q, q_pos, ws, S, s, cus, dry);
      KVQ_MHA_LUT_PG(128, 3, 2) KVQ_MHA_LUT_PG(128, 3, 4) KVQ_MHA_LUT_PG(128, 2, 2) KVQ_MHA_LUT_PG(128, 2, 4)
      KVQ_MHA_LUT_PG(64, 3, 2) KVQ_MHA_LUT_PG(64, 3, 4) KVQ_MHA_LUT_PG(64, 2, 2) KVQ_MHA_LUT_PG(64, 2, 4)
#undef KVQ_MHA_LUT_PG
      return hipErrorNotSupported;
    }
    if (g.k_mode != 0 || KB != 4) return hipErrorNotSupported;
#define KVQ_MHA_PG(bk, vb)                                                                       \
  if (BK == bk && VB == vb) {                                                                    \
    if (ko == 2) return launch_mha_typed<128, bk, 4, vb, 2, true>(c, q, q_pos, ws, S, s, cus, dry); \
    if (ko == 1) return launch_mha_typed<128, bk, 4, vb, 1, true>(c, q, q_pos, ws, S, s, cus, dry); \
    return launch_mha_typed<128, bk, 4, vb, 0, true>(c, q, q_pos, ws, S, s, cus, dry);              \
  }
    KVQ_MHA_PG(128, 4) KVQ_MHA_PG(128, 2) KVQ_MHA_PG(64, 4) KVQ_MHA_PG(64, 2)
#undef KVQ_MHA_PG
    return hipErrorNotSupported;
  }
  if (g.k_mode == 1) {
    // codebook keys: 2- and 3-bit codes (pair tables of 16 and 64 entries), no outliers
    if (ko != 0 || (KB != 3 && KB != 2)) return hipErrorNotSupported;
#define KVQ_MHA_LUT(d, bk, kb, vb) \
  if (D == d && BK == bk && KB == kb && VB == vb) return launch_mha_lut_typed<d, bk, kb, vb>(c, q, q_pos, ws, S, s, cus, dry);
    KVQ_MHA_LUT(128, 128, 3, 2) KVQ_MHA_LUT(128, 128, 3, 4) KVQ_MHA_LUT(128, 128, 2, 2) KVQ_MHA_LUT(128, 128, 2, 4)
    KVQ_MHA_LUT(128, 64, 3, 2) KVQ_MHA_LUT(128, 64, 3, 4) KVQ_MHA_LUT(128, 64, 2, 2) KVQ_MHA_LUT(128, 64, 2, 4)
    KVQ_MHA_LUT(64, 128, 3, 2) KVQ_MHA_LUT(64, 128, 3, 4) KVQ_MHA_LUT(64, 128, 2, 2) KVQ_MHA_LUT(64, 128, 2, 4)
    KVQ_MHA_LUT(64, 64, 3, 2) KVQ_MHA_LUT(64, 64, 3, 4) KVQ_MHA_LUT(64, 64, 2, 2) KVQ_MHA_LUT(64, 64, 2, 4)
#undef KVQ_MHA_LUT
    return hipErrorNotSupported;
  }
  if (g.k_mode != 0 || (KB != 4 && KB != 2)) return hipErrorNotSupported;
#define KVQ_MHA(d, bk, kb, vb)                                                                  \
  if (D == d && BK == bk && KB == kb && VB == vb) {                                             \
    if (ko == 2) return launch_mha_typed<d, bk, kb, vb, 2>(c, q, q_pos, ws, S, s, cus, dry);         \
    if (ko == 1) return launch_mha_typed<d, bk, kb, vb, 1>(c, q, q_pos, ws, S, s, cus, dry);         \
    return launch_mha_typed<d, bk, kb, vb, 0>(c, q, q_pos, ws, S, s, cus, dry);                      \
  }
  KVQ_MHA(128, 128, 4, 4) KVQ_MHA(128, 128, 4, 2) KVQ_MHA(128, 128, 2, 4) KVQ_MHA(128, 128, 2, 2)
  KVQ_MHA(128, 64, 4, 4) KVQ_MHA(128, 64, 4, 2) KVQ_MHA(128, 64, 2, 4) KVQ_MHA(128, 64, 2, 2)
  KVQ_MHA(64, 128, 4, 4) KVQ_MHA(64, 128, 4, 2) KVQ_MHA(64, 128, 2, 4) KVQ_MHA(64, 128, 2, 2)
  KVQ_MHA(64, 64, 4, 4) KVQ_MHA(64, 64, 4, 2) KVQ_MHA(64, 64, 2, 4) KVQ_MHA(64, 64, 2, 2)
#undef KVQ_MHA
  return hipErrorNotSupported;
}

}  // namespace kvq
