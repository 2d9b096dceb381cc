// Block-sparse masked attention forward, bf16 inputs, CDNA4 matrix cores.
//
// What is computed (study notes "JAX 到 VLIW ... 复习笔记", sections 15 and
// 18-23; "hstu_ops.py" (RecML) for the metadata walk, the element masks and
// the pointwise variant):
//   for each (b, h, q block i):
//     m = -inf, L = 0, O = 0
//     for each non-empty kv block j, reached through data_next:
//       S = scale * Q_i K_jᵀ                  (element mask only if class 1)
//       softmax:   m' = max(m, rowmax S), alpha = e^{m - m'}, P = e^{S - m'},
//                  L = alpha L + rowsum P, O = alpha O + P V_j
//       pointwise: P = silu(S) / q_len (masked -> 0), O = O + P V_j
//     O_i = O / L (softmax; 0 where L = 0) or O (pointwise)
//
// Work decomposition: one workgroup of NW wavefronts per (b, h, i); each
// wavefront owns 32 query rows (block_q = 32 * NW). The kv axis is walked in
// tiles of 64 keys staged in LDS.
//
// Matrix-core layout: scores are formed transposed, Sᵀ = K Qᵀ, with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Qᵀ held in registers for
// the whole kernel). In the 32x32 accumulator layout lane l holds column
// l % 32 (its query row) and 16 rows (keys), so row max / row sum are
// in-lane reductions plus one exchange between the two half-waves, and the
// probabilities are already in the B-operand layout of Oᵀ += Vᵀ Pᵀ, so P never
// leaves registers. The contraction index (key) order inside one MFMA is
// free; A (Vᵀ from LDS) is read in the order the accumulator gives P.

#include "internal.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KC = 64;           // keys per LDS tile
constexpr float kNegInf = -__builtin_inff();

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_xor32(float x) {
  // exchange with lane ^ 32 (the other half-wave)
  return __shfl_xor(x, 32, 64);
}

template <typename OutT>
__device__ inline void store4(OutT* dst, float a, float b, float c, float d);

template <>
__device__ inline void store4<__bf16>(__bf16* dst, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(dst) = v;
}

template <>
__device__ inline void store4<float>(float* dst, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(dst) = v;
}

template <int D, int NW, bool PW, typename OutT>
__global__ __launch_bounds__(NW * 64) void splash_fwd_bf16_kernel(FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  constexpr int LDS_STRIDE = D + 8;      // bf16 elements per LDS row (pad vs bank conflicts)
  constexpr int NS = D / 16;             // k-steps of the QKᵀ contraction
  constexpr int ND = D / 32;             // 32-wide output column blocks
  constexpr int CPR = D / 8;             // 16-byte chunks per row

  __shared__ __attribute__((aligned(16))) __bf16 sK[KC * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) __bf16 sV[KC * LDS_STRIDE];
  __shared__ int32_t sKseg[KC];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // Heavy-first order: the last query blocks (most kv blocks under causal
  // masks) of every (b, h) are dispatched first.
  const int BH = p.B * p.H;
  const int64_t lin = blockIdx.x;
  const int bh = (int)(lin % BH);
  const int i = p.nq - 1 - (int)(lin / BH);
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int hm = p.meta_heads == 1 ? 0 : h;
  const int bm = p.meta_batch == 1 ? 0 : b;
  const HeadBand band = p.band[hm];

  const __bf16* qg = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + h * p.v_sh;
  OutT* og = reinterpret_cast<OutT*>(p.o) + b * p.o_sb + h * p.o_sh;

  const int qrow = i * BQ + wave * 32 + l32;
  const bool qvalid = qrow < p.q_len;

  // Qᵀ as the B operand: lane holds Q[qrow][16 s + 8 hh + 0..7].
  bf16x8 qreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (qvalid) {
      qreg[s] = *reinterpret_cast<const bf16x8*>(qg + (int64_t)qrow * p.q_ss + 16 * s + 8 * hh);
    } else {
      for (int e = 0; e < 8; ++e) qreg[s][e] = (__bf16)0.0f;
    }
  }
  const bool has_seg = p.q_seg != nullptr;
  const int32_t my_qseg = (has_seg && qvalid) ? p.q_seg[(int64_t)b * p.q_len + qrow] : 0;

  f32x16 oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.0f;
  float m_run = kNegInf;   // running max of the scaled scores (log2 domain)
  float l_run = 0.0f;      // this lane's share of the running denominator

  const int64_t mrow = (((int64_t)bm * p.meta_heads + hm) * p.nq + i) * p.nk;
  const int8_t* bmask = p.block_mask + mrow;
  const int32_t* dnext = p.data_next + mrow;

  // data_next is only followed forward and within [0, nk], so any metadata
  // content ends the walk in bounds.
  int j = p.nk > 0 ? dnext[0] : p.nk;
  if (j < 0 || j > p.nk) j = p.nk;
  while (j < p.nk) {
    const bool partial = bmask[j] == 1;
    for (int t = 0; t < p.block_kv; t += KC) {
      const int k0 = j * p.block_kv + t;
      if (k0 >= p.kv_len) break;
      __syncthreads();  // every wave is done with the previous tile
      for (int c = tid; c < KC * CPR; c += NT) {
        const int r = c / CPR;
        const int cc = c % CPR;
        const int kv = k0 + r;
        uint4 kval = {0u, 0u, 0u, 0u};
        uint4 vval = {0u, 0u, 0u, 0u};
        if (kv < p.kv_len) {
          kval = *reinterpret_cast<const uint4*>(kg + (int64_t)kv * p.k_ss + cc * 8);
          vval = *reinterpret_cast<const uint4*>(vg + (int64_t)kv * p.v_ss + cc * 8);
        }
        *reinterpret_cast<uint4*>(&sK[r * LDS_STRIDE + cc * 8]) = kval;
        *reinterpret_cast<uint4*>(&sV[r * LDS_STRIDE + cc * 8]) = vval;
      }
      if (partial && has_seg && tid < KC) {
        const int kv = k0 + tid;
        sKseg[tid] = kv < p.kv_len ? p.kv_seg[(int64_t)b * p.kv_len + kv] : 0;
      }
      __syncthreads();

      // Sᵀ tile: 64 keys x 32 queries per wave, two 32x32 accumulators.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(&sK[(32 * kb + l32) * LDS_STRIDE + 16 * s + 8 * hh]);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[kb], 0, 0, 0);
        }
      }

      // sacc[kb][r] is the score of key k0 + 32 kb + 8 (r / 4) + 4 hh + r % 4.
      float x[2][16];
      if constexpr (!PW) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          for (int r = 0; r < 16; ++r) x[kb][r] = sacc[kb][r] * p.scale_log2;
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          for (int r = 0; r < 16; ++r) x[kb][r] = sacc[kb][r] * p.scale;
      }
      if (partial) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          for (int r = 0; r < 16; ++r) {
            const int kl = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const int kv = k0 + kl;
            const int dlt = kv - qrow;
            bool ok = kv < p.kv_len && dlt >= band.lo && dlt <= band.hi;
            if (has_seg) ok = ok && (sKseg[kl] == my_qseg);
            if (!ok) x[kb][r] = PW ? 0.0f : kNegInf;
          }
      }

      bf16x8 pb[2][2];
      if constexpr (!PW) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[kb][r]);
        mx = fmaxf(mx, wave_xor32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(x[kb][r] - m_use);
            rs += e;
            pb[kb][r >> 3][r & 7] = (__bf16)e;
          }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int d = 0; d < ND; ++d)
          for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
      } else {
        constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          for (int r = 0; r < 16; ++r) {
            const float xv = x[kb][r];
            const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-xv * kLog2e));
            pb[kb][r >> 3][r & 7] = (__bf16)(xv * sg * p.inv_q_len);
          }
      }

      // Oᵀ += Vᵀ Pᵀ. Step (kb, g) contracts keys 32 kb + 16 g + 8 (e / 4) + 4 hh + e % 4.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int kbase = 32 * kb + 16 * g + 4 * hh;
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              a[e] = sV[(kbase + 8 * (e >> 2) + (e & 3)) * LDS_STRIDE + 32 * d + l32];
            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][g], oacc[d], 0, 0, 0);
          }
        }
    }
    const int jn = (j + 1 < p.nk) ? dnext[j + 1] : p.nk;
    j = (jn > j && jn <= p.nk) ? jn : p.nk;
  }

  float inv = 1.0f;
  if constexpr (!PW) {
    const float l = l_run + wave_xor32(l_run);
    inv = l > 0.0f ? 1.0f / l : 0.0f;
  }
  if (qvalid) {
    OutT* orow = og + (int64_t)qrow * p.o_ss;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hh;
        store4<OutT>(orow + col, oacc[d][4 * g] * inv, oacc[d][4 * g + 1] * inv,
                     oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv);
      }
  }
}

template <int D, int NW, bool PW, typename OutT>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.nq * p.B * p.H;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((splash_fwd_bf16_kernel<D, NW, PW, OutT>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, bool PW, typename OutT>
hipError_t launch_bq(const FwdParams& p, hipStream_t stream) {
  if (p.block_q == 64) return launch_one<D, 2, PW, OutT>(p, stream);
  return launch_one<D, 4, PW, OutT>(p, stream);
}

template <bool PW, typename OutT>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  if (p.head_dim == 64) return launch_bq<64, PW, OutT>(p, stream);
  return launch_bq<128, PW, OutT>(p, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, bool pointwise, bool out_f32, hipStream_t stream) {
  if (pointwise) {
    return out_f32 ? launch_d<true, float>(p, stream) : launch_d<true, __bf16>(p, stream);
  }
  return out_f32 ? launch_d<false, float>(p, stream) : launch_d<false, __bf16>(p, stream);
}

}  // namespace splash
