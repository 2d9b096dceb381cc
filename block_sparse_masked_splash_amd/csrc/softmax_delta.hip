// delta = rowsum(O * dO) for the softmax backward: with P the row softmax
// and dP = dO Vᵀ, the softmax derivative is dS = P (dP - sum_j P_j dP_j), and
// sum_j P_j dP_j = dO · (P V) = dO · O. One pass over O and dO (memory-bound):
// each row is read by D * elem / 16 adjacent lanes with 16-byte loads, and
// summed with lane exchanges.

#include "internal.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void softmax_delta_kernel(DeltaParams p, int64_t rows) {
  constexpr int EPL = 16 / sizeof(T);  // elements per lane
  constexpr int TPR = D / EPL;         // lanes per row (a power of two, at most 32)
  const int64_t row = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.0f;
  const bool valid = row < rows;
  int64_t b = 0, h = 0, i = 0;
  if (valid) {
    i = row % p.q_len;
    const int64_t bh = row / p.q_len;
    h = bh % p.H;
    b = bh / p.H;
    const T* orow = reinterpret_cast<const T*>(p.o) + b * p.o_sb + h * p.o_sh + i * p.o_ss + part * EPL;
    const T* drow = reinterpret_cast<const T*>(p.d_o) + b * p.do_sb + h * p.do_sh + i * p.do_ss + part * EPL;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(orow);
      const bf16x8 c = *reinterpret_cast<const bf16x8*>(drow);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)c[e], acc);
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(orow);
      const f32x4 c = *reinterpret_cast<const f32x4*>(drow);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(a[e], c[e], acc);
    }
  }
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (valid && part == 0) p.delta[b * p.d_sb + h * p.d_sh + i] = acc;
}

template <typename T, int D>
hipError_t launch(const DeltaParams& p, hipStream_t stream) {
  constexpr int TPR = D / (16 / sizeof(T));
  const int64_t rows = (int64_t)p.B * p.H * p.q_len;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows * TPR + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((softmax_delta_kernel<T, D>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_delta(const DeltaParams& p, bool bf16, hipStream_t stream) {
  if (bf16) return p.head_dim == 64 ? launch<__bf16, 64>(p, stream) : launch<__bf16, 128>(p, stream);
  return p.head_dim == 64 ? launch<float, 64>(p, stream) : launch<float, 128>(p, stream);
}

}  // namespace splash
