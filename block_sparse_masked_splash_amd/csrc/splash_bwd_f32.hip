// Attention backward (pointwise SiLU and softmax) for fp32 inputs, on the
// vector ALUs in fp32 throughout.
//
// Same arithmetic and walks as the bf16 kernels ("hstu_ops.py" (RecML),
// _pointwise_splash_attention_bwd_kernel_impl): with x = scale q·k and
// sig = logistic(x) (0 where masked), p' = x sig, ds' = dp (sig + p' (1 - sig)),
// dp = dO·v; dV = sum p' dO / q_len, dK = scale sum ds' q / q_len,
// dQ = scale sum ds' k / q_len. dK and dV: one workgroup per (b, K/V head,
// kv block), walking the block's column of q blocks for every query head of
// the group; dQ: one workgroup per (b, query head, q block), walking its row
// of kv blocks. D / 32 adjacent lanes share one key (or query) row, each
// holding 32 of its head dimensions. Softmax (SM): P = e^(x - LSE),
// dS = P (dp - delta), dV = sum P dO, dK = scale sum dS q, dQ = scale sum dS k,
// with the forward's per-row LSE and delta = rowsum(dO * O).

#include "internal.h"

namespace splash {
namespace {

constexpr int TT = 32;  // rows per LDS tile

template <int G>
__device__ inline float group_sum(float x) {
  if constexpr (G >= 2) x += __shfl_xor(x, 1, 64);
  if constexpr (G >= 4) x += __shfl_xor(x, 2, 64);
  return x;
}

__device__ inline float logistic(float x) { return 1.0f / (1.0f + expf(-x)); }

template <int D, int BKV, bool SM>
__global__ __launch_bounds__(BKV*(D / 32)) void bwd_dkv_f32_kernel(BwdParams p) {
  constexpr int G = D / 32;
  constexpr int NT = BKV * G;
  constexpr int STRIDE = D + 4;
  __shared__ __attribute__((aligned(16))) float sQ[TT * STRIDE];
  __shared__ __attribute__((aligned(16))) float sO[TT * STRIDE];
  __shared__ int32_t sQseg[TT];
  __shared__ float sLse[TT];
  __shared__ float sDelta[TT];

  const int tid = threadIdx.x;
  const int rl = tid / G;
  const int part = tid % G;
  const int64_t lin = blockIdx.x;
  const int j = (int)(lin % p.c_nk);
  const int bhk = (int)(lin / p.c_nk);
  const int b = bhk / p.kv_heads;
  const int hk = bhk % p.kv_heads;
  const int bm = p.meta_batch == 1 ? 0 : b;
  const bool has_seg = p.q_seg != nullptr;

  const int key = j * BKV + rl;
  const bool kvalid = key < p.kv_len;
  const float* kr = reinterpret_cast<const float*>(p.k) + b * p.k_sb + hk * p.k_sh + (int64_t)key * p.k_ss;
  const float* vr = reinterpret_cast<const float*>(p.v) + b * p.v_sb + hk * p.v_sh + (int64_t)key * p.v_ss;
  float kv[32], vv[32], dk[32], dv[32];
  for (int d = 0; d < 32; ++d) {
    kv[d] = kvalid ? kr[part * 32 + d] : 0.0f;
    vv[d] = kvalid ? vr[part * 32 + d] : 0.0f;
    dk[d] = 0.0f;
    dv[d] = 0.0f;
  }
  const int32_t kseg = (has_seg && kvalid) ? p.kv_seg[(int64_t)b * p.kv_len + key] : 0;

  for (int g = 0; g < p.kv_group; ++g) {
    const int h = hk * p.kv_group + g;
    const int hm = p.c_meta_heads == 1 ? 0 : h;
    const HeadBand band = p.band[p.band_heads == 1 ? 0 : h];
    // the dK/dV metadata is stored by columns: this column's c_nq entries
    const int64_t col = (((int64_t)bm * p.c_meta_heads + hm) * p.c_nk + j) * p.c_nq;
    const float* qg = reinterpret_cast<const float*>(p.q) + b * p.q_sb + h * p.q_sh;
    const float* og = reinterpret_cast<const float*>(p.d_o) + b * p.do_sb + h * p.do_sh;
    // data_next only moves forward within [0, nq]
    int i = p.c_nq > 0 ? p.c_data_next[col] : p.c_nq;
    if (i < 0 || i > p.c_nq) i = p.c_nq;
    while (i < p.c_nq) {
      const bool partial = p.c_block_mask[col + i] == 1;
      // dense mask: this key's bit column of the block's entry (0 if none)
      const uint32_t* dcol = nullptr;
      if (partial && p.c_mask_blocks != nullptr) {
        int m = p.c_mask_next[col + i];
        m = m < 0 ? 0 : (m >= p.c_num_mask_blocks ? (int)p.c_num_mask_blocks - 1 : m);  // stays in the store
        dcol = p.c_mask_blocks + (int64_t)m * p.c_block_q * (p.c_block_kv / 32) + rl / 32;
      }
      for (int t = 0; t < p.c_block_q; t += TT) {
        const int q0 = i * p.c_block_q + t;
        if (q0 >= p.q_len) break;
        __syncthreads();
        for (int c = tid; c < TT * (D / 4); c += NT) {
          const int r = c / (D / 4);
          const int cc = c % (D / 4);
          const int q = q0 + r;
          float4 a = {0.f, 0.f, 0.f, 0.f}, o = {0.f, 0.f, 0.f, 0.f};
          if (q < p.q_len) {
            a = *reinterpret_cast<const float4*>(qg + (int64_t)q * p.q_ss + cc * 4);
            o = *reinterpret_cast<const float4*>(og + (int64_t)q * p.do_ss + cc * 4);
          }
          *reinterpret_cast<float4*>(&sQ[r * STRIDE + cc * 4]) = a;
          *reinterpret_cast<float4*>(&sO[r * STRIDE + cc * 4]) = o;
        }
        if (partial && has_seg && tid < TT) {
          const int q = q0 + tid;
          sQseg[tid] = q < p.q_len ? p.q_seg[(int64_t)b * p.q_len + q] : 0;
        }
        if (SM && tid < TT) {
          const int q = q0 + tid;
          const int64_t off = b * p.st_sb + h * p.st_sh + q;
          sLse[tid] = q < p.q_len ? p.lse[off] : 0.0f;
          sDelta[tid] = q < p.q_len ? p.delta[off] : 0.0f;
        }
        __syncthreads();
        for (int qq = 0; qq < TT; ++qq) {
          float s = 0.0f, dp = 0.0f;
          for (int d = 0; d < 32; ++d) {
            s = fmaf(kv[d], sQ[qq * STRIDE + part * 32 + d], s);
            dp = fmaf(vv[d], sO[qq * STRIDE + part * 32 + d], dp);
          }
          s = group_sum<G>(s);
          dp = group_sum<G>(dp);
          bool ok = true;
          if (partial) {
            const int q = q0 + qq;
            const int dlt = key - q;
            ok = kvalid && q < p.q_len && dlt >= band.lo && dlt <= band.hi && (!has_seg || sQseg[qq] == kseg);
            if (dcol != nullptr) ok = ok && ((dcol[(int64_t)(t + qq) * (p.c_block_kv / 32)] >> (rl & 31)) & 1u);
          }
          if (!ok) continue;
          const float x = s * p.scale;
          float pv, ds;
          if constexpr (SM) {
            pv = expf(x - sLse[qq]);
            ds = pv * (dp - sDelta[qq]);
          } else {
            const float sg = logistic(x);
            pv = x * sg;
            ds = dp * (sg + pv * (1.0f - sg));
          }
          for (int d = 0; d < 32; ++d) {
            dv[d] = fmaf(pv, sO[qq * STRIDE + part * 32 + d], dv[d]);
            dk[d] = fmaf(ds, sQ[qq * STRIDE + part * 32 + d], dk[d]);
          }
        }
      }
      const int in = (i + 1 < p.c_nq) ? p.c_data_next[col + i + 1] : p.c_nq;
      i = (in > i && in <= p.c_nq) ? in : p.c_nq;
    }
  }

  if (kvalid) {
    float* dkr = reinterpret_cast<float*>(p.dk) + b * p.dk_sb + hk * p.dk_sh + (int64_t)key * p.dk_ss + part * 32;
    float* dvr = reinterpret_cast<float*>(p.dv) + b * p.dv_sb + hk * p.dv_sh + (int64_t)key * p.dv_ss + part * 32;
    const float ck = SM ? p.scale : p.scale * p.inv_q_len, cv = SM ? 1.0f : p.inv_q_len;
    for (int d = 0; d < 32; ++d) {
      dkr[d] = dk[d] * ck;
      dvr[d] = dv[d] * cv;
    }
  }
}

// Rows of a q block per dQ workgroup: all of them, up to 512 threads (a q
// block of 256 rows at D = 128 takes two workgroups: 1024 threads would
// leave 128 registers per lane and spill).
template <int D, int BQ>
constexpr int dq_f32_rows() {
  return BQ * (D / 32) > 512 ? 512 / (D / 32) : BQ;
}

template <int D, int BQ, bool SM>
__global__ __launch_bounds__((dq_f32_rows<D, BQ>() * (D / 32))) void bwd_dq_f32_kernel(BwdParams p) {
  constexpr int G = D / 32;
  constexpr int ROWS = dq_f32_rows<D, BQ>();
  constexpr int SUB = BQ / ROWS;  // workgroups per q block
  constexpr int NT = ROWS * G;
  constexpr int STRIDE = D + 4;
  __shared__ __attribute__((aligned(16))) float sK[TT * STRIDE];
  __shared__ __attribute__((aligned(16))) float sV[TT * STRIDE];
  __shared__ int32_t sKseg[TT];

  const int tid = threadIdx.x;
  const int part = tid % G;
  const int BH = p.B * p.H;
  const int64_t lin = blockIdx.x;
  const int bh = (int)(lin % BH);
  const int64_t rest = lin / BH;
  const int i = p.nq - 1 - (int)(rest / SUB);
  const int rl = tid / G + (int)(rest % SUB) * ROWS;  // row within the q block
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int hk = h / p.kv_group;
  const int hm = p.meta_heads == 1 ? 0 : h;
  const int bm = p.meta_batch == 1 ? 0 : b;
  const HeadBand band = p.band[p.band_heads == 1 ? 0 : h];
  const bool has_seg = p.q_seg != nullptr;

  const float* kg = reinterpret_cast<const float*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const float* vg = reinterpret_cast<const float*>(p.v) + b * p.v_sb + hk * p.v_sh;
  const int qrow = i * BQ + rl;
  const bool qvalid = qrow < p.q_len;
  const float* qr = reinterpret_cast<const float*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)qrow * p.q_ss;
  const float* orr = reinterpret_cast<const float*>(p.d_o) + b * p.do_sb + h * p.do_sh + (int64_t)qrow * p.do_ss;
  float qv[32], ov[32], dq[32];
  for (int d = 0; d < 32; ++d) {
    qv[d] = qvalid ? qr[part * 32 + d] : 0.0f;
    ov[d] = qvalid ? orr[part * 32 + d] : 0.0f;
    dq[d] = 0.0f;
  }
  const int32_t qseg = (has_seg && qvalid) ? p.q_seg[(int64_t)b * p.q_len + qrow] : 0;
  float lse = 0.0f, dlt = 0.0f;
  if (SM && qvalid) {
    lse = p.lse[b * p.st_sb + h * p.st_sh + qrow];
    dlt = p.delta[b * p.st_sb + h * p.st_sh + qrow];
  }

  const int64_t mrow = (((int64_t)bm * p.meta_heads + hm) * p.nq + i) * p.nk;
  int jb = p.nk > 0 ? p.data_next[mrow] : p.nk;
  if (jb < 0 || jb > p.nk) jb = p.nk;
  while (jb < p.nk) {
    const bool partial = p.block_mask[mrow + jb] == 1;
    // dense mask: this query's row of the block's entry (0 if none)
    const uint32_t* drow = nullptr;
    if (partial && p.mask_blocks != nullptr) {
      int m = p.mask_next[mrow + jb];
      m = m < 0 ? 0 : (m >= p.num_mask_blocks ? (int)p.num_mask_blocks - 1 : m);  // stays in the store
      drow = p.mask_blocks + ((int64_t)m * BQ + rl) * (p.block_kv / 32);
    }
    for (int t = 0; t < p.block_kv; t += TT) {
      const int k0 = jb * p.block_kv + t;
      if (k0 >= p.kv_len) break;
      __syncthreads();
      for (int c = tid; c < TT * (D / 4); c += NT) {
        const int r = c / (D / 4);
        const int cc = c % (D / 4);
        const int kk = k0 + r;
        float4 a = {0.f, 0.f, 0.f, 0.f}, o = {0.f, 0.f, 0.f, 0.f};
        if (kk < p.kv_len) {
          a = *reinterpret_cast<const float4*>(kg + (int64_t)kk * p.k_ss + cc * 4);
          o = *reinterpret_cast<const float4*>(vg + (int64_t)kk * p.v_ss + cc * 4);
        }
        *reinterpret_cast<float4*>(&sK[r * STRIDE + cc * 4]) = a;
        *reinterpret_cast<float4*>(&sV[r * STRIDE + cc * 4]) = o;
      }
      if (partial && has_seg && tid < TT) {
        const int kk = k0 + tid;
        sKseg[tid] = kk < p.kv_len ? p.kv_seg[(int64_t)b * p.kv_len + kk] : 0;
      }
      __syncthreads();
      for (int kk = 0; kk < TT; ++kk) {
        float s = 0.0f, dp = 0.0f;
        for (int d = 0; d < 32; ++d) {
          s = fmaf(qv[d], sK[kk * STRIDE + part * 32 + d], s);
          dp = fmaf(ov[d], sV[kk * STRIDE + part * 32 + d], dp);
        }
        s = group_sum<G>(s);
        dp = group_sum<G>(dp);
        bool ok = true;
        if (partial) {
          const int key = k0 + kk;
          const int dlt = key - qrow;
          ok = qvalid && key < p.kv_len && dlt >= band.lo && dlt <= band.hi && (!has_seg || sKseg[kk] == qseg);
          if (drow != nullptr) ok = ok && ((drow[(t + kk) >> 5] >> ((t + kk) & 31)) & 1u);
        }
        if (!ok) continue;
        const float x = s * p.scale;
        float ds;
        if constexpr (SM) {
          ds = expf(x - lse) * (dp - dlt);
        } else {
          const float sg = logistic(x);
          ds = dp * (sg + x * sg * (1.0f - sg));
        }
        for (int d = 0; d < 32; ++d) dq[d] = fmaf(ds, sK[kk * STRIDE + part * 32 + d], dq[d]);
      }
    }
    const int jn = (jb + 1 < p.nk) ? p.data_next[mrow + jb + 1] : p.nk;
    jb = (jn > jb && jn <= p.nk) ? jn : p.nk;
  }

  if (qvalid) {
    float* dqr = reinterpret_cast<float*>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)qrow * p.dq_ss + part * 32;
    const float cq = SM ? p.scale : p.scale * p.inv_q_len;
    for (int d = 0; d < 32; ++d) dqr[d] = dq[d] * cq;
  }
}

template <int D, int BKV, bool SM>
hipError_t launch_dkv_f32(const BwdParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.B * p.kv_heads * p.c_nk;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkv_f32_kernel<D, BKV, SM>), dim3((unsigned)grid), dim3(BKV * (D / 32)), 0, stream, p);
  return hipGetLastError();
}

template <int D, int BQ, bool SM>
hipError_t launch_dq_f32(const BwdParams& p, hipStream_t stream) {
  constexpr int ROWS = dq_f32_rows<D, BQ>();
  const int64_t grid = (int64_t)p.nq * p.B * p.H * (BQ / ROWS);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<D, BQ, SM>), dim3((unsigned)grid), dim3(ROWS * (D / 32)), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool SM>
hipError_t launch_sm_f32(const BwdParams& p, hipStream_t stream) {
  hipError_t e = p.c_block_kv == 64 ? launch_dkv_f32<D, 64, SM>(p, stream) : launch_dkv_f32<D, 128, SM>(p, stream);
  if (e != hipSuccess) return e;
  if (p.block_q == 64) return launch_dq_f32<D, 64, SM>(p, stream);
  if (p.block_q == 256) return launch_dq_f32<D, 256, SM>(p, stream);
  return launch_dq_f32<D, 128, SM>(p, stream);
}

template <int D>
hipError_t launch_d_f32(const BwdParams& p, hipStream_t stream) {
  return p.softmax ? launch_sm_f32<D, true>(p, stream) : launch_sm_f32<D, false>(p, stream);
}

}  // namespace

hipError_t launch_pointwise_bwd_f32(const BwdParams& p, hipStream_t stream) {
  return p.head_dim == 64 ? launch_d_f32<64>(p, stream) : launch_d_f32<128>(p, stream);
}

}  // namespace splash
