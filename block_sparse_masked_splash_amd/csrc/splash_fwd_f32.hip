// Block-sparse masked attention forward for fp32 inputs, on the vector ALUs
// in fp32 (no bf16 rounding anywhere).
//
// Same walk as the bf16 kernel (study notes "JAX 到 VLIW ... 复习笔记",
// sections 15 and 18-21; "hstu_ops.py" (RecML) _next_nonzero / _apply_mask /
// pointwise forward): one workgroup per (b, h, q block), kv blocks reached
// through data_next, element mask only on class-1 blocks, online softmax
// per kv tile of 32 keys. Each query row is owned by D/32 adjacent lanes,
// each holding 32 of the head dimensions of q and of the accumulator. With a
// dense mask, a partial block's bits (its entry of the mask store) are ANDed
// into the element mask.

#include "internal.h"

namespace splash {
namespace {

constexpr int KT = 32;  // keys per LDS tile
constexpr float kNegInf = -__builtin_inff();

template <int G>
__device__ inline float group_sum(float x) {
  if constexpr (G >= 2) x += __shfl_xor(x, 1, 64);
  if constexpr (G >= 4) x += __shfl_xor(x, 2, 64);
  return x;
}

// Rows of a q block per workgroup: all of them, up to 512 threads (a q block
// of 256 rows at D = 128 takes two workgroups: 1024 threads would leave 128
// registers per lane and spill).
template <int D, int BQ>
constexpr int f32_rows() {
  return BQ * (D / 32) > 512 ? 512 / (D / 32) : BQ;
}

template <int D, int BQ, bool PW>
__global__ __launch_bounds__((f32_rows<D, BQ>() * (D / 32))) void splash_fwd_f32_kernel(FwdParams p) {
  constexpr int G = D / 32;
  constexpr int ROWS = f32_rows<D, BQ>();
  constexpr int SUB = BQ / ROWS;  // workgroups per q block
  constexpr int NT = ROWS * G;
  constexpr int STRIDE = D + 4;
  __shared__ __attribute__((aligned(16))) float sK[KT * STRIDE];
  __shared__ __attribute__((aligned(16))) float sV[KT * STRIDE];
  __shared__ int32_t sKseg[KT];

  const int tid = threadIdx.x;
  const int rl0 = tid / G;
  const int part = tid % G;

  const int BH = p.B * p.H;
  const int64_t lin = blockIdx.x;
  const int bh = (int)(lin % BH);
  const int64_t rest = lin / BH;
  const int i = p.nq - 1 - (int)(rest / SUB);
  const int rl = rl0 + (int)(rest % SUB) * ROWS;  // row within the q block
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int hm = p.meta_heads == 1 ? 0 : h;
  const int bm = p.meta_batch == 1 ? 0 : b;
  const HeadBand band = p.band[p.band_heads == 1 ? 0 : h];

  const float* qg = reinterpret_cast<const float*>(p.q) + b * p.q_sb + h * p.q_sh;
  const int hk = h / p.kv_group;  // K/V head read by query head h
  const float* kg = reinterpret_cast<const float*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const float* vg = reinterpret_cast<const float*>(p.v) + b * p.v_sb + hk * p.v_sh;
  float* og = reinterpret_cast<float*>(p.o) + b * p.o_sb + h * p.o_sh;

  const int qrow = i * BQ + rl;
  const bool qvalid = qrow < p.q_len;
  float qv[32], o[32];
  for (int d = 0; d < 32; ++d) {
    qv[d] = qvalid ? qg[(int64_t)qrow * p.q_ss + part * 32 + d] : 0.0f;
    o[d] = 0.0f;
  }
  const bool has_seg = p.q_seg != nullptr;
  const int32_t my_qseg = (has_seg && qvalid) ? p.q_seg[(int64_t)b * p.q_len + qrow] : 0;
  float m_run = kNegInf, l_run = 0.0f;

  const int64_t mrow = (((int64_t)bm * p.meta_heads + hm) * p.nq + i) * p.nk;
  const int8_t* bmask = p.block_mask + mrow;
  const int32_t* dnext = p.data_next + mrow;

  // data_next is only followed forward and within [0, nk], so any metadata
  // content ends the walk in bounds.
  int j = p.nk > 0 ? dnext[0] : p.nk;
  if (j < 0 || j > p.nk) j = p.nk;
  const bool dense = p.mask_blocks != nullptr;
  const int wpr = p.block_kv / 32;
  while (j < p.nk) {
    const bool partial = bmask[j] == 1;
    // dense mask: this row's bits of block j (row i * BQ + rl of the block store entry)
    const uint32_t* drow = nullptr;
    if (partial && dense) {
      int m = p.mask_next[mrow + j];
      m = m < 0 ? 0 : (m >= p.num_mask_blocks ? (int)p.num_mask_blocks - 1 : m);  // any content stays in the store
      drow = p.mask_blocks + ((int64_t)m * p.block_q + rl) * wpr;
    }
    for (int t = 0; t < p.block_kv; t += KT) {
      const int k0 = j * p.block_kv + t;
      if (k0 >= p.kv_len) break;
      __syncthreads();
      // the tile's K and V rows: every load of the thread is issued before
      // the first LDS store, so their latencies overlap
      constexpr int PER = KT * (D / 4) / NT;  // float4 of K (and of V) per thread
      static_assert(PER * NT == KT * (D / 4), "tile not divisible over the threads");
      float4 kval[PER], vval[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int c = tid + u * NT;
        const int kv = k0 + c / (D / 4);
        kval[u] = vval[u] = float4{0.f, 0.f, 0.f, 0.f};
        if (kv < p.kv_len) {
          kval[u] = *reinterpret_cast<const float4*>(kg + (int64_t)kv * p.k_ss + (c % (D / 4)) * 4);
          vval[u] = *reinterpret_cast<const float4*>(vg + (int64_t)kv * p.v_ss + (c % (D / 4)) * 4);
        }
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int c = tid + u * NT;
        *reinterpret_cast<float4*>(&sK[(c / (D / 4)) * STRIDE + (c % (D / 4)) * 4]) = kval[u];
        *reinterpret_cast<float4*>(&sV[(c / (D / 4)) * STRIDE + (c % (D / 4)) * 4]) = vval[u];
      }
      if (partial && has_seg && tid < KT) {
        const int kv = k0 + tid;
        sKseg[tid] = kv < p.kv_len ? p.kv_seg[(int64_t)b * p.kv_len + kv] : 0;
      }
      __syncthreads();

      float s[KT];
      for (int kk = 0; kk < KT; ++kk) {
        float acc = 0.0f;
        for (int d = 0; d < 32; ++d) acc = fmaf(qv[d], sK[kk * STRIDE + part * 32 + d], acc);
        s[kk] = group_sum<G>(acc) * p.scale;
      }
      // whether this row may see key k0 + kk (every key of a full block)
      auto allowed = [&](int kk) -> bool {
        if (!partial) return true;
        const int kv = k0 + kk;
        const int dlt = kv - qrow;
        bool ok = kv < p.kv_len && dlt >= band.lo && dlt <= band.hi && (!has_seg || sKseg[kk] == my_qseg);
        if (drow != nullptr) ok = ok && ((drow[(t + kk) >> 5] >> ((t + kk) & 31)) & 1u);
        return ok;
      };
      if constexpr (PW) {
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
          // (a key a row may not see is passed over, as in the softmax below;
          // the branch also keeps the compiler from loading the V rows of
          // many keys ahead, which ran it out of registers)
          if (!allowed(kk)) continue;
          // silu(s) / q_len; the reciprocal instruction is within 1 ulp
          const float pr = s[kk] * __builtin_amdgcn_rcpf(1.0f + expf(-s[kk])) * p.inv_q_len;
          for (int d = 0; d < 32; ++d) o[d] = fmaf(pr, sV[kk * STRIDE + part * 32 + d], o[d]);
        }
      } else {
        float mx = kNegInf;
        for (int kk = 0; kk < KT; ++kk)
          if (allowed(kk)) mx = fmaxf(mx, s[kk]);
        const float m_new = fmaxf(m_run, mx);
        if (m_new != kNegInf) {
          const float alpha = expf(m_run - m_new);
          l_run *= alpha;
          for (int d = 0; d < 32; ++d) o[d] *= alpha;
          for (int kk = 0; kk < KT; ++kk) {
            if (!allowed(kk)) continue;
            const float e = expf(s[kk] - m_new);
            l_run += e;
            for (int d = 0; d < 32; ++d) o[d] = fmaf(e, sV[kk * STRIDE + part * 32 + d], o[d]);
          }
          m_run = m_new;
        }
      }
    }
    const int jn = (j + 1 < p.nk) ? dnext[j + 1] : p.nk;
    j = (jn > j && jn <= p.nk) ? jn : p.nk;
  }

  if (qvalid) {
    float inv = 1.0f;
    if constexpr (!PW) inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    // log-sum-exp of the row's scores (-inf with no allowed key)
    if constexpr (!PW)
      if (p.lse != nullptr && part == 0)
        p.lse[b * p.lse_sb + h * p.lse_sh + qrow] = l_run > 0.0f ? m_run + logf(l_run) : kNegInf;
    float* orow = og + (int64_t)qrow * p.o_ss + part * 32;
    for (int d = 0; d < 32; ++d) orow[d] = o[d] * inv;
  }
}

template <int D, int BQ, bool PW>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  constexpr int ROWS = f32_rows<D, BQ>();
  const int64_t grid = (int64_t)p.nq * p.B * p.H * (BQ / ROWS);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((splash_fwd_f32_kernel<D, BQ, PW>), dim3((unsigned)grid), dim3(ROWS * (D / 32)), 0,
                     stream, p);
  return hipGetLastError();
}

template <bool PW>
hipError_t launch_pw(const FwdParams& p, hipStream_t stream) {
  if (p.head_dim == 64) {
    if (p.block_q == 256) return launch_one<64, 256, PW>(p, stream);
    return p.block_q == 64 ? launch_one<64, 64, PW>(p, stream) : launch_one<64, 128, PW>(p, stream);
  }
  if (p.block_q == 256) return launch_one<128, 256, PW>(p, stream);
  return p.block_q == 64 ? launch_one<128, 64, PW>(p, stream) : launch_one<128, 128, PW>(p, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, bool pointwise, hipStream_t stream) {
  return pointwise ? launch_pw<true>(p, stream) : launch_pw<false>(p, stream);
}

}  // namespace splash
