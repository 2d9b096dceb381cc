// Block metadata: class of every (batch, head, q block, kv block) and the
// index of the next non-empty kv block.
//
// "hstu_ops.py" (RecML), _next_nonzero: a block runs when its class is > 0 and
// needs no element mask when its class is not 1; the kv block fetched at grid
// step j is data_next[h, i, j]. Study notes "JAX 到 VLIW ... 复习笔记",
// section 21: a fully masked kv block is skipped by pointing at the next
// valid one, so it is never loaded.
//
// Classes: 0 = no allowed pair, 2 = every pair of the (bq x bkv) block allowed,
// 1 otherwise; pairs past the sequence ends count as not allowed.
//
// One wavefront per metadata row (bm, hm, i). The row is walked back to front
// in chunks of 64 kv blocks: each lane classifies one block, a ballot marks
// the non-empty ones, and each lane's data_next is the lowest marked block at
// or after it, else the carry from the chunks already done.

#include "internal.h"

namespace splash {
namespace {

__device__ inline int64_t clamp_count(int64_t lo, int64_t hi) { return hi >= lo ? hi - lo + 1 : 0; }

// Class of block (i, j) for head band `hb`, batch row b (segments only).
__device__ int classify(const MaskInfoParams& p, HeadBand hb, int b, int i, int j) {
  const int64_t q_begin = (int64_t)i * p.block_q;
  const int64_t k_begin = (int64_t)j * p.block_kv;
  const int64_t k_end = k_begin + p.block_kv - 1;               // inclusive
  const int64_t k_last = k_end < p.kv_len - 1 ? k_end : (int64_t)p.kv_len - 1;
  bool any_in = false;
  bool any_out = (q_begin + p.block_q > p.q_len) || (k_end >= p.kv_len);
  for (int r = 0; r < p.block_q; ++r) {
    const int64_t q = q_begin + r;
    if (q >= p.q_len) break;
    int64_t a = q + hb.lo;
    int64_t z = q + hb.hi;
    if (a < k_begin) a = k_begin;
    if (z > k_last) z = k_last;
    const int64_t n = clamp_count(a, z);
    if (n < p.block_kv) any_out = true;
    if (n == 0) {
      if (any_in && any_out) return 1;
      continue;
    }
    if (p.q_seg == nullptr) {
      any_in = true;
    } else {
      const int32_t qs = p.q_seg[(int64_t)b * p.q_len + q];
      const int32_t* ks = p.kv_seg + (int64_t)b * p.kv_len;
      for (int64_t k = a; k <= z; ++k) {
        if (ks[k] == qs) any_in = true; else any_out = true;
        if (any_in && any_out) return 1;
      }
    }
    if (any_in && any_out) return 1;
  }
  if (!any_in) return 0;
  return any_out ? 1 : 2;
}

__global__ __launch_bounds__(256) void mask_info_kernel(MaskInfoParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)p.meta_batch * p.meta_heads * p.nq;
  if (row >= rows) return;
  const int i = (int)(row % p.nq);
  const int hm = (int)((row / p.nq) % p.meta_heads);
  const int bm = (int)(row / ((int64_t)p.nq * p.meta_heads));
  const HeadBand hb = p.band[hm];
  int8_t* bmask = p.block_mask + row * p.nk;
  int32_t* dnext = p.data_next + row * p.nk;
  int carry = p.nk;
  const int nchunks = (p.nk + 63) / 64;
  for (int c = nchunks - 1; c >= 0; --c) {
    const int j = c * 64 + lane;
    int cls = 0;
    if (j < p.nk) {
      cls = classify(p, hb, bm, i, j);
      bmask[j] = (int8_t)cls;
    }
    const uint64_t bits = __ballot(cls != 0);
    const uint64_t at_or_after = bits >> lane;
    if (j < p.nk) dnext[j] = at_or_after ? j + __builtin_ctzll(at_or_after) : carry;
    if (bits) carry = c * 64 + __builtin_ctzll(bits);
  }
}

}  // namespace

hipError_t launch_mask_info(const MaskInfoParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.meta_batch * p.meta_heads * p.nq;
  if (rows == 0 || p.nk == 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(mask_info_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace splash
