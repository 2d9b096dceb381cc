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
// The causal / window part of a head's mask is a band k - q in [lo, hi] with
// lo <= 0 <= hi, so its class has a closed form per block. Segment ids are
// arbitrary integers: where they are given, each q block and kv block is first
// reduced to its runs of equal ids, and an entry whose two blocks have few
// runs is classified from the rectangles those runs form, each with one id on
// either side, by the band's closed form; other entries compare all their
// pairs (the segment path below).
// data_next is then a suffix scan of each metadata row, one wavefront per
// row: the row is walked back to front in chunks of 64 kv blocks, a ballot
// marks the non-empty ones, and each lane takes the lowest marked block at or
// after it, else the carry from the chunks already done.
//
// The dK/dV pass of the pointwise backward walks columns instead ("hstu_ops.py",
// _pointwise_splash_attention_bwd_kernel: grid over kv blocks, then heads,
// then q steps; _next_nonzero(next_i=True) reads data_next[h, i, j] as the
// q block to fetch). Its metadata has the same classes, and data_next of
// (i, j) is the first non-empty q block at or after i in column j (nq if
// none); it is stored by columns, [meta_batch, meta_heads, nk, nq].

#include "internal.h"

namespace splash {
namespace {

struct BlockSpan {
  int64_t q0, q1;  // first and last valid query of the block
  int64_t k0, k1;  // first and last valid key
  bool ragged;     // the block reaches past a sequence end
};

__device__ inline BlockSpan block_span(const MaskInfoParams& p, int i, int j) {
  BlockSpan s;
  s.q0 = (int64_t)i * p.block_q;
  s.k0 = (int64_t)j * p.block_kv;
  const int64_t qe = s.q0 + p.block_q, ke = s.k0 + p.block_kv;
  s.q1 = (qe < p.q_len ? qe : (int64_t)p.q_len) - 1;
  s.k1 = (ke < p.kv_len ? ke : (int64_t)p.kv_len) - 1;
  s.ragged = qe > p.q_len || ke > p.kv_len;
  return s;
}

// Class of a block under the band alone. Some query q of the block sees a key
// of the block iff q + lo <= k1 and q + hi >= k0 for a q in [q0, q1]; every
// pair is allowed iff the band of the last query starts at or before k0 and
// the band of the first query ends at or after k1 (and nothing is ragged).
__device__ inline int band_class(const BlockSpan& s, HeadBand hb) {
  const int64_t qa = s.q0 > s.k0 - hb.hi ? s.q0 : s.k0 - hb.hi;
  const int64_t qb = s.q1 < s.k1 - hb.lo ? s.q1 : s.k1 - hb.lo;
  if (qa > qb) return 0;
  const bool full = !s.ragged && s.q1 + hb.lo <= s.k0 && s.q0 + hb.hi >= s.k1;
  return full ? 2 : 1;
}

__device__ inline void decode_row(const MaskInfoParams& p, int64_t row, int& bm, int& hm, int& i) {
  i = (int)(row % p.nq);
  hm = (int)((row / p.nq) % p.meta_heads);
  bm = (int)(row / ((int64_t)p.nq * p.meta_heads));
}

// Segment path: one workgroup per metadata entry (grid-stride over entries).
// The id ranges of the block's queries and keys decide most blocks without a
// pair test: disjoint ranges share no id (class 0), and a single common id
// leaves the band to decide. Otherwise every pair is tested.
constexpr int kSegThreads = 256;

__device__ inline int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int w = __shfl_xor(v, o, 64);
    v = w < v ? w : v;
  }
  return v;
}
__device__ inline int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

__global__ __launch_bounds__(kSegThreads) void segment_class_kernel(MaskInfoParams p, int64_t entries) {
  __shared__ int32_t qs[1024];
  __shared__ int32_t ks[1024];
  __shared__ int32_t red[4][kSegThreads / 64];  // per wave: q min, q max, k min, k max
  const int t = threadIdx.x;
  const int wv = t >> 6;
  for (int64_t e0 = blockIdx.x; e0 < entries; e0 += gridDim.x) {
    const int64_t row = e0 / p.nk;
    const int j = (int)(e0 - row * p.nk);
    int bm, hm, i;
    decode_row(p, row, bm, hm, i);
    // where this entry's class goes: row layout e0, column layout its transpose
    const int64_t e = p.columns ? (((int64_t)bm * p.meta_heads + hm) * p.nk + j) * p.nq + i : e0;
    const HeadBand hb = p.band[hm];
    const BlockSpan s = block_span(p, i, j);
    const int base = band_class(s, hb);
    if (base == 0) {
      if (t == 0) p.block_mask[e] = 0;
      continue;
    }
    const int nvq = (int)(s.q1 - s.q0 + 1), nvk = (int)(s.k1 - s.k0 + 1);
    const int32_t* qrow = p.q_seg + (int64_t)bm * p.q_len + s.q0;
    const int32_t* krow = p.kv_seg + (int64_t)bm * p.kv_len + s.k0;
    __syncthreads();  // the previous entry's readers are done with qs, ks and red
    int qmin = 0x7fffffff, qmax = (int)0x80000000, kmin = 0x7fffffff, kmax = (int)0x80000000;
    for (int r = t; r < nvq; r += kSegThreads) {
      const int v = qrow[r];
      qs[r] = v;
      qmin = v < qmin ? v : qmin;
      qmax = v > qmax ? v : qmax;
    }
    for (int c = t; c < nvk; c += kSegThreads) {
      const int v = krow[c];
      ks[c] = v;
      kmin = v < kmin ? v : kmin;
      kmax = v > kmax ? v : kmax;
    }
    qmin = wave_min(qmin);
    qmax = wave_max(qmax);
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if ((t & 63) == 0) {
      red[0][wv] = qmin;
      red[1][wv] = qmax;
      red[2][wv] = kmin;
      red[3][wv] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSegThreads / 64; ++w) {
      qmin = red[0][w] < qmin ? red[0][w] : qmin;
      qmax = red[1][w] > qmax ? red[1][w] : qmax;
      kmin = red[2][w] < kmin ? red[2][w] : kmin;
      kmax = red[3][w] > kmax ? red[3][w] : kmax;
    }
    if (qmax < kmin || kmax < qmin) {  // no id in common
      if (t == 0) p.block_mask[e] = 0;
      continue;
    }
    if (qmin == qmax && kmin == kmax) {  // one id on both sides
      if (t == 0) p.block_mask[e] = (int8_t)base;
      continue;
    }
    // Pair test, in chunks of up to 256 key columns: thread t takes column
    // t % span of the chunk and every (256 / span)-th row.
    int any_in = 0, any_out = 0;
    for (int c0 = 0; c0 < nvk; c0 += kSegThreads) {
      const int span = nvk - c0 < kSegThreads ? nvk - c0 : kSegThreads;
      const int rstep = kSegThreads / span;
      const int r0 = t / span;
      if (r0 < rstep) {
        const int c = c0 + (t - r0 * span);
        const int32_t kid = ks[c];
        const int64_t d0 = (s.k0 + c) - s.q0;  // k - q at row 0
        for (int r = r0; r < nvq; r += rstep) {
          const int64_t d = d0 - r;
          const bool allowed = d >= hb.lo && d <= hb.hi && qs[r] == kid;
          any_in |= allowed;
          any_out |= !allowed;
        }
      }
    }
    any_in = __syncthreads_or(any_in);
    any_out = __syncthreads_or(any_out);
    if (t == 0) p.block_mask[e] = (int8_t)(!any_in ? 0 : (any_out || base == 1 ? 1 : 2));
  }
}

// Segment path for metadata large enough to lend scratch, in two launches
// before the scan. First, one wavefront per q block and per kv block of each
// batch row records the block's runs of equal ids (the positions where the id
// changes, and the ids), up to kMaxRuns of them, into the data_next buffer
// (the scan overwrites it afterwards). Then one lane per metadata entry: when
// both blocks have at most kMaxRuns runs, the block splits into rectangles of
// one q run by one kv run, each with a single id on either side, so its class
// follows from the band's closed form on those rectangles (a rectangle whose
// two ids differ allows nothing). Packed documents longer than a block give
// at most two runs per block. An entry with a block of more runs is tested
// pair by pair by its whole wavefront.
constexpr int kMaxRuns = 4;
constexpr int kRunWords = 1 + 2 * kMaxRuns;  // run count (kMaxRuns + 1: more), starts, ids

__host__ __device__ inline int64_t segment_run_words(const MaskInfoParams& p) {
  return (int64_t)kRunWords * p.B * (p.nq + p.nk);
}

// record of q block i (or kv block j) of batch row b
__device__ inline const int32_t* run_record(const MaskInfoParams& p, const int32_t* runs, bool isq, int b, int blk) {
  const int64_t idx = isq ? (int64_t)b * p.nq + blk : (int64_t)p.B * p.nq + (int64_t)b * p.nk + blk;
  return runs + idx * kRunWords;
}

__global__ __launch_bounds__(256) void segment_runs_kernel(MaskInfoParams p, int32_t* runs) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nqb = (int64_t)p.B * p.nq, nkb = (int64_t)p.B * p.nk;
  if (w >= nqb + nkb) return;
  const bool isq = w < nqb;
  const int64_t idx = isq ? w : w - nqb;
  const int nb = isq ? p.nq : p.nk;
  const int b = (int)(idx / nb), blk = (int)(idx - (int64_t)b * nb);
  const int bs = isq ? p.block_q : p.block_kv;
  const int len = isq ? p.q_len : p.kv_len;
  const int32_t* ids = (isq ? p.q_seg : p.kv_seg) + (int64_t)b * len + (int64_t)blk * bs;
  const int n = len - blk * bs < bs ? len - blk * bs : bs;  // valid positions of the block
  int32_t* rec = runs + (w * kRunWords);
  int count = 0;
  for (int r0 = 0; r0 < n && count <= kMaxRuns; r0 += 64) {
    const int r = r0 + lane;
    const bool in = r < n;
    const int v = in ? ids[r] : 0;
    const int prev = (in && r > 0) ? ids[r - 1] : 0;
    const bool start = in && (r == 0 || prev != v);
    const uint64_t m = __ballot(start);
    if (start) {
      const int slot = count + __builtin_popcountll(m & ((1ull << lane) - 1));
      if (slot < kMaxRuns) {
        rec[1 + slot] = r;
        rec[1 + kMaxRuns + slot] = v;
      }
    }
    count += __builtin_popcountll(m);
  }
  if (lane == 0) rec[0] = count <= kMaxRuns ? count : kMaxRuns + 1;
}

// Class contribution of the rectangles of block (i, j) from the two blocks'
// run records (each at most kMaxRuns runs): whether some allowed pair exists
// and whether some pair is not allowed. Positions are absolute.
__device__ inline void runs_class(const int32_t* qr, const int32_t* kr, int64_t q0, int64_t q1, int64_t k0,
                                  int64_t k1, HeadBand hb, bool& any_in, bool& any_out) {
  const int nqr = qr[0], nkr = kr[0];
  any_in = false;
  any_out = false;
  for (int a = 0; a < nqr; ++a) {
    const int64_t qa = q0 + qr[1 + a];
    const int64_t qb = a + 1 < nqr ? q0 + qr[2 + a] - 1 : q1;
    const int qid = qr[1 + kMaxRuns + a];
    for (int c = 0; c < nkr; ++c) {
      const int64_t ka = k0 + kr[1 + c];
      const int64_t kb = c + 1 < nkr ? k0 + kr[2 + c] - 1 : k1;
      if (qid != kr[1 + kMaxRuns + c]) {
        any_out = true;  // different ids: nothing in this rectangle is allowed
        continue;
      }
      // the band on the rectangle [qa, qb] x [ka, kb], as band_class
      const int64_t lo_q = qa > ka - hb.hi ? qa : ka - hb.hi;
      const int64_t hi_q = qb < kb - hb.lo ? qb : kb - hb.lo;
      if (lo_q <= hi_q) any_in = true;
      if (!(qb + hb.lo <= ka && qa + hb.hi >= kb)) any_out = true;
    }
  }
}

// Pair test of block (i, j) of batch row b by one wavefront: whether some
// pair the band allows has equal ids, and whether some pair is not allowed.
// Lane L takes keys L, L + 64, ...; the block's query ids go round the
// wavefront 64 at a time and are read back one per step with a lane read.
__device__ inline int segment_pair_class(const MaskInfoParams& p, int b, int i, int j, HeadBand hb, int base,
                                         int lane) {
  const BlockSpan s = block_span(p, i, j);
  const int q0 = (int)s.q0, k0 = (int)s.k0;
  const int nvq = (int)(s.q1 - s.q0 + 1), nvk = (int)(s.k1 - s.k0 + 1);
  const int32_t* qrow = p.q_seg + (int64_t)b * p.q_len + q0;
  const int32_t* krow = p.kv_seg + (int64_t)b * p.kv_len + k0;
  bool any_in = false, any_out = false;
  for (int c0 = 0; c0 < nvk; c0 += 64) {
    const int c = c0 + lane;
    const bool kvalid = c < nvk;
    const int kid = kvalid ? krow[c] : 0;
    for (int r0 = 0; r0 < nvq; r0 += 64) {
      const int qv_lane = r0 + lane < nvq ? qrow[r0 + lane] : 0;
      const int rn = nvq - r0 < 64 ? nvq - r0 : 64;
      for (int rr = 0; rr < rn; ++rr) {
        const int qid = __builtin_amdgcn_readlane(qv_lane, rr);
        const int d = (k0 + c) - (q0 + r0 + rr);
        const bool allowed = d >= hb.lo && d <= hb.hi && kid == qid;
        any_in |= kvalid & allowed;
        any_out |= kvalid & !allowed;
      }
    }
  }
  const bool in = __ballot(any_in) != 0, out = __ballot(any_out) != 0;
  return !in ? 0 : (out || base == 1 ? 1 : 2);
}

__global__ __launch_bounds__(256) void segment_classify_kernel(MaskInfoParams p, const int32_t* runs) {
  const int lane = threadIdx.x & 63;
  // a line is a metadata row (row layout) or column (column layout); a
  // wavefront takes 64 consecutive entries of one line, a lane each
  const int across = p.columns ? p.nk : p.nq;  // lines per (batch, head)
  const int line_len = p.columns ? p.nq : p.nk;
  const int64_t chunks = (line_len + 63) / 64;
  const int64_t lines = (int64_t)p.meta_batch * p.meta_heads * across;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= lines * chunks) return;
  const int64_t line = w / chunks;
  const int pos = (int)(w - line * chunks) * 64 + lane;
  const int other = (int)(line % across);
  const int hm = (int)((line / across) % p.meta_heads);
  const int bm = (int)(line / ((int64_t)across * p.meta_heads));
  const int i = p.columns ? pos : other;
  const int j = p.columns ? other : pos;
  const bool valid = pos < line_len;
  const HeadBand hb = p.band[hm];
  int cls = 0, base = 0;
  bool pair = false;
  if (valid) {
    const BlockSpan sp = block_span(p, i, j);
    base = band_class(sp, hb);
    if (base != 0) {
      const int32_t* qr = run_record(p, runs, true, bm, i);
      const int32_t* kr = run_record(p, runs, false, bm, j);
      if (qr[0] <= kMaxRuns && kr[0] <= kMaxRuns) {
        bool any_in, any_out;
        runs_class(qr, kr, sp.q0, sp.q1, sp.k0, sp.k1, hb, any_in, any_out);
        cls = !any_in ? 0 : (any_out || base == 1 ? 1 : 2);
      } else {
        pair = true;
      }
    }
  }
  // entries with a block of many runs: the whole wavefront tests each one
  uint64_t todo = __ballot(pair);
  while (todo) {
    const int src = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int spos = pos - lane + src;
    const int si = p.columns ? spos : i, sj = p.columns ? j : spos;
    const int sbase = __builtin_amdgcn_readlane(base, src);
    const int c = segment_pair_class(p, bm, si, sj, hb, sbase, lane);
    if (lane == src) cls = c;
  }
  if (valid) p.block_mask[line * line_len + pos] = (int8_t)cls;
}

// One wavefront per metadata row: classes (closed form, or read back from the
// segment pass) and the data_next suffix scan.
template <bool kFromSegments>
__global__ __launch_bounds__(256) void row_scan_kernel(MaskInfoParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)p.meta_batch * p.meta_heads * p.nq;
  if (row >= rows) return;
  int bm, hm, i;
  decode_row(p, row, bm, hm, i);
  const HeadBand hb = p.band[hm];
  int8_t* bmask = p.block_mask + row * p.nk;
  int32_t* dnext = p.data_next + row * p.nk;
  int carry = p.nk;
  const int nchunks = (p.nk + 63) / 64;
  for (int c = nchunks - 1; c >= 0; --c) {
    const int j = c * 64 + lane;
    int cls = 0;
    if (j < p.nk) {
      if constexpr (kFromSegments) {
        cls = bmask[j];
      } else {
        cls = band_class(block_span(p, i, j), hb);
        bmask[j] = (int8_t)cls;
      }
    }
    const uint64_t bits = __ballot(cls != 0);
    const uint64_t at_or_after = bits >> lane;
    if (j < p.nk) dnext[j] = at_or_after ? j + __builtin_ctzll(at_or_after) : carry;
    if (bits) carry = c * 64 + __builtin_ctzll(bits);
  }
}

// Column walk of the dK/dV pass, in the column layout: one wavefront per
// (metadata batch, head, kv block) column, with the classes (closed form, or
// read back from the segment pass) and the same back-to-front ballot scan
// over its q blocks. A column's entries are contiguous, so the dK/dV kernel's
// walk reads consecutive metadata, as the forward's does along a row.
template <bool kFromSegments>
__global__ __launch_bounds__(256) void column_scan_kernel(MaskInfoParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t col = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t cols = (int64_t)p.meta_batch * p.meta_heads * p.nk;
  if (col >= cols) return;
  const int j = (int)(col % p.nk);
  const int hm = (int)((col / p.nk) % p.meta_heads);
  const HeadBand hb = p.band[hm];
  int8_t* bmask = p.block_mask + col * p.nq;
  int32_t* dnext = p.data_next + col * p.nq;
  int carry = p.nq;
  const int nchunks = (p.nq + 63) / 64;
  for (int c = nchunks - 1; c >= 0; --c) {
    const int i = c * 64 + lane;
    int cls = 0;
    if (i < p.nq) {
      if constexpr (kFromSegments) {
        cls = bmask[i];
      } else {
        cls = band_class(block_span(p, i, j), hb);
        bmask[i] = (int8_t)cls;
      }
    }
    const uint64_t bits = __ballot(cls != 0);
    const uint64_t at_or_after = bits >> lane;
    if (i < p.nq) dnext[i] = at_or_after ? i + __builtin_ctzll(at_or_after) : carry;
    if (bits) carry = c * 64 + __builtin_ctzll(bits);
  }
}

// Classes of every entry with segment ids, before the scan (lines = rows or
// columns of the metadata, line_len entries each). Metadata too small to
// hold the blocks' run records in its data_next buffer takes the
// one-workgroup-per-entry kernel instead.
hipError_t launch_segment_classes(const MaskInfoParams& p, int64_t lines, int line_len, hipStream_t stream) {
  const int64_t entries = lines * line_len;
  if (entries < segment_run_words(p)) {
    const int64_t grid = entries < (1 << 20) ? entries : (1 << 20);
    hipLaunchKernelGGL(segment_class_kernel, dim3((unsigned)grid), dim3(kSegThreads), 0, stream, p, entries);
    return hipGetLastError();
  }
  const int64_t block_waves = (int64_t)p.B * (p.nq + p.nk);
  hipLaunchKernelGGL(segment_runs_kernel, dim3((unsigned)((block_waves + 3) / 4)), dim3(256), 0, stream, p,
                     p.data_next);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = lines * ((line_len + 63) / 64);
  hipLaunchKernelGGL(segment_classify_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, p,
                     p.data_next);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mask_info_dkv(const MaskInfoParams& p, hipStream_t stream) {
  const int64_t cols = (int64_t)p.meta_batch * p.meta_heads * p.nk;
  if (cols == 0 || p.nq == 0) return hipSuccess;
  const int64_t blocks = (cols + 3) / 4;
  if (p.q_seg != nullptr) {
    const hipError_t e = launch_segment_classes(p, cols, p.nq, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(column_scan_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(column_scan_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_mask_info(const MaskInfoParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.meta_batch * p.meta_heads * p.nq;
  if (rows == 0 || p.nk == 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  if (p.q_seg != nullptr) {
    const hipError_t e = launch_segment_classes(p, rows, p.nk, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(row_scan_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(row_scan_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace splash
