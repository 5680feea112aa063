// quantize.hip -- append-time sequencing of the block quantizer (keys and values,
// quantize_block.h), the tail copy and the rotary tables.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {


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

// ---------------------------------------------------------------- tail copy
// The new tokens that stay unquantized, rows src0.. of the input, to tail slots dst0..
// In a paged cache each sequence derives both from its own length (read before the
// lengths advance).
__global__ void tail_copy_kernel(kvq_cache c, const uint16_t* __restrict__ k_new,
                                 const uint16_t* __restrict__ v_new, int64_t n_new, int64_t src0_arg,
                                 int64_t dst0_arg, const int64_t* __restrict__ n_seq) {
  const int D = c.cfg.head_dim, Bk = c.cfg.k_block;
  const int64_t bh = blockIdx.y;
  int64_t src0 = src0_arg, dst0 = dst0_arg, count = n_new;  // n_new: the input's rows per sequence
  if (c.seq_lens) {
    const int64_t b = bh / c.cfg.kv_heads;
    count = n_seq ? min(max(n_seq[b], (int64_t)0), n_new) : n_new;
    const int64_t L0 = seq_len_of(c, b), L1 = L0 + count;
    const int64_t nf0 = L0 / Bk, nf1 = L1 / Bk, rem = L1 - nf1 * Bk;
    if (rem == 0) return;
    src0 = count - (nf1 > nf0 ? rem : count);
    dst0 = nf1 > nf0 ? 0 : L0 - nf0 * Bk;
  }
  const int64_t rows = count - src0;
  const int64_t chunks_per_row = D / 8;
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

// ---------------------------------------------------------------- paged lengths
__global__ void seq_lens_add_kernel(int64_t* lens, int batch, int64_t n, int set, const int64_t* n_seq) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) lens[b] = set ? n : lens[b] + (n_seq ? n_seq[b] : n);
}

}  // namespace

hipError_t launch_seq_lens_add(const kvq_cache& c, int64_t n, hipStream_t s, const int64_t* n_seq) {
  const int B = c.cfg.batch;
  hipLaunchKernelGGL(seq_lens_add_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, c.seq_lens, B, n, 0,
                     n_seq);
  return hipGetLastError();
}

hipError_t launch_seq_lens_set(const kvq_cache& c, int64_t n, hipStream_t s) {
  const int B = c.cfg.batch;
  hipLaunchKernelGGL(seq_lens_add_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, c.seq_lens, B, n, 1,
                     (const int64_t*)nullptr);
  return hipGetLastError();
}

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
                           hipStream_t s, const int64_t* n_seq) {
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  if (c.cfg.k_mode == 2) return launch_quantize_fp8(c, k_new, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
  hipError_t e = c.cfg.k_mode == 1
                     ? launch_quantize_keys_lut(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s)
                     : launch_quantize_keys_uniform(c, k_new, old_len, n_new, n_first, nblocks, n_seq, s);
  if (e != hipSuccess) return e;
  return launch_quantize_values(c, v_new, old_len, n_new, n_first, nblocks, n_seq, s);
}

hipError_t launch_tail_copy(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                            int64_t n_new, int64_t src0, int64_t dst0, hipStream_t s, const int64_t* n_seq) {
  const int64_t BH = (int64_t)c.cfg.batch * c.cfg.kv_heads;
  if (BH > 65535) return hipErrorInvalidValue;
  // a paged cache: at most Bk - 1 rows per sequence, each sequence's own
  const int64_t rows = c.seq_lens ? (n_new < c.cfg.k_block ? n_new : (int64_t)c.cfg.k_block) : n_new - src0;
  const int64_t work = rows * (c.cfg.head_dim / 8) * 2;
  const int blocks = (int)((work + 255) / 256 < 64 ? (work + 255) / 256 : 64);
  hipLaunchKernelGGL(tail_copy_kernel, dim3(blocks > 0 ? blocks : 1, (unsigned)BH), dim3(256), 0, s,
                     c, k_new, v_new, n_new, src0, dst0, n_seq);
  return hipGetLastError();
}

}  // namespace kvq
