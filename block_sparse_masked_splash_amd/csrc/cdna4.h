// Device helpers shared by the CDNA4 (gfx950) attention kernels: vector
// types, direct HBM -> LDS tile copies through buffer resources, waits and
// barriers, scalar-cache metadata reads, the LDS swizzle and vector stores.
#pragma once

#include "internal.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
struct bf16x2x4 {
  bf16x2 v[4];
};
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// Kinds of element mask a kernel instance applies on partial blocks: the
// head's band only, the band and segment ids, or the band and a dense mask's
// stored bits (segment ids given with a dense mask are folded into its
// metadata, so the kernels never see both); kAnyMask decides at run time
// from the parameters (one instance for every kind).
enum MaskKind { kBandOnly = 0, kSegments = 1, kDense = 2, kAnyMask = 3 };

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// {x, x of lane ^ 32}: the gfx950 half-wave swap returns both halves' values
// in each lane, in an order that does not matter for max and sum.
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct HBM -> LDS copies through a buffer resource: every active lane
// fetches 16 (or 4) bytes at byte offset voff of the buffer, and lane L's
// bytes land at LDS byte address lds + 16 L (4 L). Offsets at or past the
// buffer's size read as zero, which clips a tile at the end of the sequence
// with no per-lane arithmetic. The hardware range check covers the VGPR
// offset (plus the instruction offset) only, not the SGPR offset, so every
// part of a lane's offset travels in voff and the SGPR offset is 0. Issued
// through asm so that the compiler does not treat the tile being filled as a
// pending write to every LDS read that follows; completion is awaited
// explicitly with wait_vmcnt. The copies set m0 (the LDS destination) and
// name it as clobbered; the compiler warns that it does not preserve a
// reserved register across such a statement. That is safe here because
// nothing of the compiler's lives in m0 in these kernels: on this target LDS
// instructions do not read it, and the kernels use none of the instructions
// that do (no builtin LDS-direct loads, no indexed register moves, no GWS).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kRawBufferWord3 = 0x00020000u;  // 32-bit data format, no swizzle, no stride

__device__ inline u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kRawBufferWord3;
  return r;
}
__device__ inline void lds_copy4(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds)
               : "memory", "m0");
}
// N 16-byte-per-lane copies of row groups: copy n reads the buffer at the
// lane's byte offset vo[n] (its whole offset, range-checked) and writes LDS
// lds0 + n * LSTEP (64 lanes x 16 bytes each). m0 advances inside one asm
// block, so no per-copy LDS address is kept live.
#define SPLASH_COPY1(V)                                         \
  "s_nop 0\n\t"                                                 \
  "buffer_load_dwordx4 " V ", %[rs], 0 offen lds\n\t"          \
  "s_add_u32 m0, m0, %[ls]\n\t"
template <int N, int LSTEP>
__device__ inline void lds_copy_rows(u32x4 rsrc, const uint32_t (&vo)[N], uint32_t lds0) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "copy count");
  if constexpr (N == 1) {
    asm volatile("s_mov_b32 m0, %[lds]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[v0], %[rs], 0 offen lds"
                 :
                 : [lds] "s"(lds0), [rs] "s"(rsrc), [v0] "v"(vo[0])
                 : "memory", "m0");
  } else if constexpr (N == 2) {
    asm volatile("s_mov_b32 m0, %[lds]\n\t" SPLASH_COPY1("%[v0]") SPLASH_COPY1("%[v1]")
                 :
                 : [lds] "s"(lds0), [rs] "s"(rsrc), [ls] "i"(LSTEP), [v0] "v"(vo[0]), [v1] "v"(vo[1])
                 : "memory", "m0", "scc");
  } else if constexpr (N == 4) {
    asm volatile("s_mov_b32 m0, %[lds]\n\t" SPLASH_COPY1("%[v0]") SPLASH_COPY1("%[v1]")
                     SPLASH_COPY1("%[v2]") SPLASH_COPY1("%[v3]")
                 :
                 : [lds] "s"(lds0), [rs] "s"(rsrc), [ls] "i"(LSTEP), [v0] "v"(vo[0]), [v1] "v"(vo[1]),
                   [v2] "v"(vo[2]), [v3] "v"(vo[3])
                 : "memory", "m0", "scc");
  } else {
    asm volatile("s_mov_b32 m0, %[lds]\n\t" SPLASH_COPY1("%[v0]") SPLASH_COPY1("%[v1]")
                     SPLASH_COPY1("%[v2]") SPLASH_COPY1("%[v3]")
                         SPLASH_COPY1("%[v4]") SPLASH_COPY1("%[v5]")
                             SPLASH_COPY1("%[v6]") SPLASH_COPY1("%[v7]")
                 :
                 : [lds] "s"(lds0), [rs] "s"(rsrc), [ls] "i"(LSTEP), [v0] "v"(vo[0]), [v1] "v"(vo[1]),
                   [v2] "v"(vo[2]), [v3] "v"(vo[3]), [v4] "v"(vo[4]), [v5] "v"(vo[5]), [v6] "v"(vo[6]),
                   [v7] "v"(vo[7])
                 : "memory", "m0", "scc");
  }
}
#undef SPLASH_COPY1

// LDS byte address of a (wave-uniform) shared-memory pointer, as an SGPR value.
__device__ inline uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p);
}

// Workgroup barrier without a memory fence: LDS reads are complete once their
// values have been consumed, and direct-load completion is tracked by vmcnt,
// so no wait on outstanding global traffic is wanted here.
__device__ inline void barrier_only() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unconstrained
  __builtin_amdgcn_s_barrier();
}

// Metadata is read-only for the whole launch and its addresses are uniform
// across the workgroup: read it through the constant address space so the
// loads go through the scalar cache (SGPRs, lgkmcnt) and never wait behind
// the tile copies on vmcnt.
typedef __attribute__((address_space(4))) const uint32_t* const_u32_ptr;
__device__ inline int scalar_load_i32(const int32_t* p) {
  return (int)*(const_u32_ptr)(uintptr_t)p;
}
// The kernel's parameter block read in place in the kernarg segment (P must
// be the kernel's first argument). The pointer is opaque to the optimizer,
// so fields read through it are loaded where they are used instead of being
// held in scalar registers for the kernel's lifetime: for values that only a
// rare path needs.
template <typename P>
__device__ inline const __attribute__((address_space(4))) P* kernarg_params() {
  auto ptr = (const __attribute__((address_space(4))) P*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ptr));
  return ptr;
}
// Class of kv block j in a metadata row, read as part of its aligned 32-bit
// word (block_mask buffers are padded to whole words).
__device__ inline int block_class(const int8_t* row, int j) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(row + j);
  const uint32_t w = *(const_u32_ptr)(a & ~(uintptr_t)3);
  return (int)((w >> (8 * (a & 3))) & 0xffu);
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

// LDS chunk position of logical 16-byte chunk c of tile row r (64 banks of
// 4 bytes). Two access patterns must be free of bank conflicts:
//   * row operand reads (ds_read_b128, 16 lanes per pass): rows r .. r + 15
//     at one logical chunk must land on 16 distinct 4-bank groups;
//   * transposing reads (ds_read_b64_tr_b16, 32 lanes per pass): rows
//     4m .. 4m + 3, each at the 4 chunks of one 64-byte head-dim span, must
//     cover all 64 banks.
// A 128-dim row spans all 64 banks: XOR with r & 15 (bits swapped in pairs)
// gives 16 distinct positions per 16 rows and keeps a 4-chunk span whole. A
// 64-dim row spans half of them (rows of one parity share a half): the XOR
// takes row bits 1-3, bit 1 onto chunk bit 2 so that rows 4m and 4m + 2 use
// opposite 4-chunk halves, bits 2-3 onto chunk bits 0-1.
template <int D>
__device__ constexpr int swz(int c, int r) {
  if constexpr (D == 128) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
}


// ---- row-major LDS tiles of D bf16 per row, chunks swizzled by swz ----

// Operand read from 32 tile rows (starting at a multiple of 16): lane
// (l32, hh) takes row l32, logical 16-byte chunk 2 s + hh, i.e. head-dim
// 16 s + 8 hh .. + 7 of that row: the A operand of a 32x32x16 product with
// the rows as M (or, identically laid out, a B operand with the rows as N).
template <int D>
__device__ inline void row_operand_offsets(int lane, int (&off)[D / 16]) {
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) off[s] = l32 * (D * 2) + 16 * swz<D>(2 * s + hh, l32);
}

// Transposing reads (ds_read_b64_tr_b16) of 16 tile rows for the A operand of
// C[d x n] += Xᵀ[d x rows] P[rows x n], where P is a 32x32 accumulator turned
// into a B operand: its lane (n, hh) holds rows 16 g + {4 hh .. 4 hh + 3} and
// 16 g + 8 + {4 hh .. 4 hh + 3} for g = 0 (elements 0-7) and 1 (8-15). Lane L
// reads 4 values of row 8 half + 4 hh + ((L % 16) >> 2) at head-dim
// 32 db + 16 ((L >> 4) & 1) + 4 (L & 3); a row offset of 16 g does not change
// the swizzle.
template <int D>
__device__ inline void transpose_operand_offsets(int lane, int (&off)[2][D / 32]) {
  const int hh = lane >> 5;
  const int rsub = 4 * hh + ((lane & 15) >> 2);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dcol = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      const int row = 8 * half + rsub;
      off[half][db] = row * (D * 2) + 16 * swz<D>(dcol >> 3, row) + 2 * (dcol & 7);
    }
}

// Global byte offsets of the direct copies that fill a tile of rows. Copy n
// of wave w covers rows (n NW + w) RPI .. + RPI - 1 (RPI = 64 / (D / 8) rows
// per copy instruction); lane L writes row RPI (n NW + w) + L / CPR at chunk
// position L % CPR, so it fetches the logical chunk stored there. The swizzle
// only sees row & 15, so the chunk choice only depends on (n NW + w) & 3.
// Each offset is the lane's whole byte offset from the tile's first row, so
// the buffer's range check clips every row past the end of the sequence.
template <int D, int NW, int LOADS>
__device__ inline void tile_copy_offsets(int lane, int wave, int64_t row_bytes, uint32_t (&sel)[LOADS]) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  uint32_t vo[4];
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    const int rr = lane / CPR;
    const int row = v4 * RPI + rr;
    int chunk = 0;
    for (int cc = 0; cc < CPR; ++cc)  // logical chunk at position lane % CPR
      if (swz<D>(cc, row) == lane % CPR) chunk = cc;
    vo[v4] = (uint32_t)(rr * row_bytes + chunk * 16);
  }
#pragma unroll
  for (int n = 0; n < LOADS; ++n)
    sel[n] = vo[(n * NW + wave) & 3] + (uint32_t)((n * NW + wave) * RPI * row_bytes);
}

}  // namespace
}  // namespace splash
