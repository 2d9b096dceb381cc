// Softmax attention forward at head_dim 128 with 64 query rows per
// wavefront: the same computation as splash_fwd_bf16_kernel (study notes
// "JAX 到 VLIW ... 复习笔记", sections 15 and 18-23; "hstu_ops.py" for the
// metadata walk and the element masks), with each K and V operand read from
// LDS feeding the matrix products of two 32-row blocks instead of one.
//
// Why: the forward's LDS traffic costs matrix throughput on this chip (an
// MFMA loop with the forward's operand reads runs 15-20% below the same loop
// on register operands, and issuing the reads a whole step ahead does not
// help; the tile copies into LDS cost the one-block kernel 12%), so halving
// both the operand reads and the copies per FLOP pays even though a
// wavefront then holds two blocks of Q, O and scores and only two
// wavefronts fit a SIMD.
//
// Work decomposition: workgroups of four wavefronts and 256 query rows (two
// query blocks of 128, or one of 256); each wavefront owns two 32-row blocks
// (rb = 0, 1). Everything else (the XCD-aware order, the data_next walk, the
// double-buffered direct HBM -> LDS tile copies of 32 keys, each now serving
// 256 rows, the transposed-score layout with P kept in registers, the
// max-free fast path of the log2-domain softmax, the band test on partial
// blocks) is the one-block forward's, per row block. Segment ids and dense
// masks take that kernel.

#include <cstdlib>
#include <type_traits>

#include "cdna4.h"

namespace splash {
namespace {

constexpr float kRescaleSlack64 = 32.0f;      // log2 units a tile max may exceed the reference by
constexpr float kFastLimit64 = 1099511627776.0f;  // 2^40 (see the forward)

// Four wavefronts of 64 rows: 256 query rows per workgroup.
struct Rows64Tiling {
  static constexpr int NW = 4;
  static constexpr int D = 128;
  static constexpr int KC = 32;                 // keys per LDS tile
  static constexpr int NT = NW * 64;            // threads
  static constexpr int ROWB = D * 2;            // bytes per key row
  static constexpr int RPI = 64 / (D / 8);      // rows written by one direct-load instruction
  static constexpr int TILE = KC * ROWB;        // bytes of one K or V tile
  static constexpr int LOADS = (KC / RPI) / NW; // direct loads per wave per matrix per tile
  static constexpr int NS = D / 16;             // k-steps of the QKᵀ contraction
  static constexpr int ND = D / 32;             // 32-wide output blocks
  static constexpr int LDS_BYTES = 2 * 2 * TILE;  // [stage][K | V][TILE]
};

// QB: metadata query blocks per workgroup. With block_q = 256 (QB = 1)
// wavefront w owns rows 64 w .. 64 w + 63 of the block. With block_q = 128
// (QB = 2) the workgroup covers query blocks 2 i and 2 i + 1, and wavefront w
// owns rows 32 w .. 32 w + 31 of each (row block rb of the wavefront lies in
// query block 2 i + rb): the kv walk is the union of the two blocks' walks,
// and a kv block empty for one of them is masked whole for its rows by the
// band test (with a band-only mask, an empty block has no pair inside the
// band and the sequence), so every wavefront does the same work.
template <int QB, typename OutT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void splash_fwd_rows64_kernel(FwdParams p, int total_work, int work_per_xcd, int units_grouped) {
  using T = Rows64Tiling;
  constexpr int NW = T::NW;
  constexpr int D = T::D;
  constexpr int KC = T::KC;
  constexpr int NS = T::NS;
  constexpr int ND = T::ND;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  // XCD-aware order, as in the forward: XCD x takes units x, x + 8, ... in
  // groups, work items heaviest first across the group's units.
  const int nitems = QB == 2 ? (p.nq + 1) / 2 : p.nq;  // workgroups per query head
  const int xcd = (int)(blockIdx.x & 7), k_in_xcd = (int)(blockIdx.x >> 3);
  const int per_unit = nitems * p.kv_group;
  int unit, rest;
  if (units_grouped) {
    const int G = units_grouped;
    const int units_xcd = (p.B * p.kv_heads) / 8;
    const int gi = k_in_xcd / (G * per_unit);
    const int g_units = units_xcd - gi * G < G ? units_xcd - gi * G : G;
    const int r = k_in_xcd - gi * G * per_unit;
    const int ri0 = r / (g_units * p.kv_group);
    const int rem = r - ri0 * g_units * p.kv_group;
    const int ug = rem / p.kv_group;
    unit = xcd + 8 * (gi * G + ug);
    rest = ri0 * p.kv_group + (rem - ug * p.kv_group);
  } else {
    const int wid = xcd * work_per_xcd + k_in_xcd;
    if (wid >= total_work) return;
    unit = wid / per_unit;
    rest = wid - unit * per_unit;
  }
  const int ri = rest / p.kv_group;
  const int item = nitems - 1 - ri;  // heaviest first under causal masks
  const int b = unit / p.kv_heads;
  const int hk = unit - b * p.kv_heads;
  const int h = hk * p.kv_group + (rest - ri * p.kv_group);
  const int hm = p.meta_heads == 1 ? 0 : h;
  const int bm = p.meta_batch == 1 ? 0 : b;
  const HeadBand band = p.band[p.band_heads == 1 ? 0 : h];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const __bf16* qg = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
  const char* kg = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + hk * p.k_sh);
  const char* vg = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + hk * p.v_sh);
  OutT* og = reinterpret_cast<OutT*>(p.o) + b * p.o_sb + h * p.o_sh;
  const int64_t k_rs = p.k_ss * 2;
  const int64_t v_rs = p.v_ss * 2;

  // ---- Q of the two row blocks (B operands of Sᵀ = K Qᵀ) ----
  const bool negate_q = p.scale < 0.0f;
  const float c = fmaxf(negate_q ? -p.scale_log2 : p.scale_log2, 1.17549435e-38f);
  int qrow[2];
  bf16x8 qreg[2][NS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    qrow[rb] = QB == 2 ? (2 * item + rb) * p.block_q + wave * 32 + l32 : item * p.block_q + wave * 64 + rb * 32 + l32;
    const bool valid = qrow[rb] < p.q_len;
    const __bf16* qrow_ptr = qg + (int64_t)(valid ? qrow[rb] : p.q_len - 1) * p.q_ss + 8 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      i16x8 v = *reinterpret_cast<const i16x8*>(qrow_ptr + 16 * s);
      if (negate_q) v ^= (short)0x8000;
      if (!valid) v = (i16x8){0, 0, 0, 0, 0, 0, 0, 0};
      qreg[rb][s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // LDS operand offsets: at D = 128 the swizzle XORs a row-dependent value
  // into the chunk index, so the K offset of k-step s is the k-step-0 offset
  // XOR 32 s, the V offset of output block db the block-0 offset XOR 64 db,
  // and the V offset of the upper 8-row half (row + 8 flips bit 1 of the
  // swizzle) the lower one XOR 32, plus 8 rows; only two base offsets are
  // kept (registers are what limits this kernel), each read forms its
  // address with one or two integer operations.
  int koff0, voff0;
  {
    int koff_all[NS];
    row_operand_offsets<D>(lane, koff_all);
    int voff_all[2][ND];
    transpose_operand_offsets<D>(lane, voff_all);
    koff0 = koff_all[0];
    voff0 = voff_all[0][0];
  }

  // Copy offsets: every copy of a wave covers row group n NW + wave, whose
  // swizzled chunk choice depends on the group mod 4 only, so with four
  // wavefronts the offsets of a wave's copies differ by 4 row groups each.
  uint32_t kvsel, vvsel;
  {
    uint32_t all_k[T::LOADS], all_v[T::LOADS];
    tile_copy_offsets<D, NW>(lane, wave, k_rs, all_k);
    tile_copy_offsets<D, NW>(lane, wave, v_rs, all_v);
    kvsel = all_k[0];
    vvsel = all_v[0];
  }
  const uint32_t k_group_step = (uint32_t)(NW * T::RPI * k_rs);
  const uint32_t v_group_step = (uint32_t)(NW * T::RPI * v_rs);

  // metadata rows: one per row block (the same row twice when QB = 1); a
  // second query block past the end has no row and is empty everywhere
  const int qblk1 = QB == 2 ? 2 * item + 1 : item;
  const bool has1 = qblk1 < p.nq;
  const int64_t mrow0 = (((int64_t)bm * p.meta_heads + hm) * p.nq + (QB == 2 ? 2 * item : item)) * p.nk;
  const int64_t mrow1 = (((int64_t)bm * p.meta_heads + hm) * p.nq + (has1 ? qblk1 : 0)) * p.nk;
  const int8_t* bmask0 = p.block_mask + mrow0;
  const int8_t* bmask1 = p.block_mask + mrow1;
  const int32_t* dnext0 = p.data_next + mrow0;
  const int32_t* dnext1 = p.data_next + mrow1;

  auto issue_tile = [&](int stage, int j, int t) {
    const int key0 = j * p.block_kv + t;
    char* kdst = smem + stage * 2 * T::TILE;
    char* vdst = kdst + T::TILE;
    const int rows = p.kv_len - key0 < KC ? p.kv_len - key0 : KC;  // rows past the end read as 0
    const u32x4 krs = buffer_rsrc(kg + key0 * k_rs, (uint32_t)(rows * k_rs));
    const u32x4 vrs = buffer_rsrc(vg + key0 * v_rs, (uint32_t)(rows * v_rs));
    uint32_t ko[T::LOADS], vo[T::LOADS];
#pragma unroll
    for (int n = 0; n < T::LOADS; ++n) {
      ko[n] = kvsel + (uint32_t)n * k_group_step;
      vo[n] = vvsel + (uint32_t)n * v_group_step;
    }
    lds_copy_rows<T::LOADS, NW * 1024>(krs, ko, lds_addr(kdst + wave * T::RPI * T::ROWB));
    lds_copy_rows<T::LOADS, NW * 1024>(vrs, vo, lds_addr(vdst + wave * T::RPI * T::ROWB));
  };

  // Walk: the union of the row blocks' walks. data_next is only followed
  // forward and within [0, nk], so any metadata content ends it in bounds.
  auto first_of = [&](const int32_t* dn) {
    int j = p.nk > 0 ? scalar_load_i32(dn) : p.nk;
    return (j < 0 || j > p.nk) ? p.nk : j;
  };
  auto next_of = [&](const int32_t* dn, int j) {
    const int jn = (j + 1 < p.nk) ? scalar_load_i32(dn + j + 1) : p.nk;
    return (jn > j && jn <= p.nk) ? jn : p.nk;
  };
  // a block's class for the two row blocks, packed (bit 0: row block 0 not
  // full, bit 1: row block 1 not full)
  auto classes = [&](int j) {
    const int c0 = block_class(bmask0, j);
    const int c1 = has1 ? block_class(bmask1, j) : 0;
    return (c0 != 2 ? 1 : 0) | (c1 != 2 ? 2 : 0);
  };
  int cur_j;
  {
    const int j0 = first_of(dnext0);
    const int j1 = has1 ? first_of(dnext1) : p.nk;
    cur_j = j0 < j1 ? j0 : j1;
  }
  int cur_t = 0;
  int cur_cls = cur_j < p.nk ? classes(cur_j) : 0;

  // zeroed tiles: rows a clipped copy leaves unwritten never hold NaN
  for (int o = tid * 16; o < T::LDS_BYTES; o += T::NT * 16)
    *reinterpret_cast<uint4*>(smem + o) = uint4{0u, 0u, 0u, 0u};
  barrier_only();

  f32x16 oacc[2][ND];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[rb][db][r] = 0.0f;
  float mref[2] = {kNegInf, kNegInf};  // per row block: reference max (log2 domain)
  float lsum[2] = {0.0f, 0.0f};        // per row block: this lane's share of L

  auto next_block = [&](int j) {
    const int n0 = next_of(dnext0, j);
    const int n1 = has1 ? next_of(dnext1, j) : p.nk;
    return n0 < n1 ? n0 : n1;
  };
  if (cur_j < p.nk) issue_tile(0, cur_j, 0);

  auto step = [&](auto stage_tag) -> bool {
    constexpr int stage = decltype(stage_tag)::value;
    int nxt_j = cur_j, nxt_t = cur_t + KC;
    int nxt_cls = cur_cls;
    if (nxt_t >= p.block_kv || cur_j * p.block_kv + nxt_t >= p.kv_len) {
      nxt_j = next_block(cur_j);
      nxt_t = 0;
      nxt_cls = nxt_j < p.nk ? classes(nxt_j) : 0;
    }
    wait_vmcnt<0>();
    barrier_only();
    __builtin_amdgcn_s_setprio(1);
    if (nxt_j < p.nk) issue_tile(stage ^ 1, nxt_j, nxt_t);

    const int k0 = cur_j * p.block_kv + cur_t;
    const int cls = cur_cls;
    const char* kt = smem + stage * 2 * T::TILE;
    const char* vt = kt + T::TILE;

    // (the bases are opaque to the compiler here, so that it forms the
    // per-read offsets in the loop instead of holding all of them)
    asm volatile("" : "+v"(koff0), "+v"(voff0), "+v"(kvsel), "+v"(vvsel));
    const int voff1 = (voff0 ^ 32) + 8 * T::ROWB;

    // ---- Sᵀ = K Qᵀ for both row blocks, each K operand read once ----
    f32x16 sacc[2];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + (koff0 ^ (32 * s)));
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        sacc[rb] = s == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[rb][s], (f32x16){}, 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[rb][s], sacc[rb], 0, 0, 0);
    }
    // Raised issue priority from the barrier through the S products (the
    // next tile's copies and both S chains), normal for the softmax and P V:
    // measured against raising it through the softmax too, equal at B=2 H=32
    // S=8192 and 2% faster on the 16 x 32768 mixed-mask workload; without
    // any raise, or raised for P V instead, 2-4% slower.
    __builtin_amdgcn_s_setprio(0);

    // ---- band mask on the row blocks for which the block is not full ----
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if (cls & (1 << rb)) {
        int a = qrow[rb] + band.lo - k0;
        int e = qrow[rb] + band.hi - k0;
        a = a > 0 ? a : 0;
        e = e < p.kv_len - 1 - k0 ? e : p.kv_len - 1 - k0;
        e = e < KC - 1 ? e : KC - 1;
        if (e < a) a = e = KC;  // no key of the tile
        const bool whole = a == 0 && e == KC - 1;
        const bool none = a == KC;
        if (__builtin_amdgcn_ballot_w64(!(whole || none)) == 0) {
          // every row keeps all 32 keys or none: one lane mask
          if (__builtin_amdgcn_ballot_w64(none) != 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[rb][r] = none ? kNegInf : sacc[rb][r];
          }
        } else {
          // (the lane's half-wave offset is formed here from the lane id
          // rather than kept live across the loop)
          const int lid = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
          const uint32_t width = (uint32_t)(e - a);
          const int base = ((lid >> 5) << 2) - a;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kc = 8 * (r >> 2) + (r & 3);
            sacc[rb][r] = (uint32_t)(base + kc) <= width ? sacc[rb][r] : kNegInf;
          }
        }
      }
    }

    // ---- probabilities, per row block (fast path and raising path) ----
    bf16x8 pb[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      auto probs = [&](float mneg) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pb[rb][r >> 3][r & 7] = (__bf16)fast_exp2(__builtin_fmaf(sacc[rb][r], c, mneg));
        float rs = 0.0f;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const bf16x2x4 pr = __builtin_bit_cast(bf16x2x4, pb[rb][g]);
#pragma unroll
          for (int u = 0; u < 4; ++u) rs = __builtin_amdgcn_fdot2_f32_bf16(pr.v[u], kOnes2, rs, false);
        }
        return rs;
      };
      float rs = probs(-mref[rb]);
      const bool fast = rs <= kFastLimit64;  // false for NaN / inf too
      if (__builtin_amdgcn_ballot_w64(!fast) != 0) {
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[rb][r]);
        mx = max_xor32(mx) * c;
        const bool raise = mx > mref[rb] + kRescaleSlack64;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          const float alpha = raise ? fast_exp2(mref[rb] - mx) : 1.0f;
          mref[rb] = raise ? mx : mref[rb];
          lsum[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha;
        }
        rs = probs(mref[rb] == kNegInf ? 0.0f : -mref[rb]);
      }
      lsum[rb] += rs;
    }

    // ---- Oᵀ += Vᵀ Pᵀ for both row blocks, each V operand read once ----
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vt + 16 * g * T::ROWB + (voff0 ^ (64 * db))));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vt + 16 * g * T::ROWB + (voff1 ^ (64 * db))));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rb][g], oacc[rb][db], 0, 0, 0);
      }
    }

    cur_j = nxt_j;
    cur_t = nxt_t;
    cur_cls = nxt_cls;
    return cur_j < p.nk;
  };
  while (cur_j < p.nk) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
  }

  // ---- O = O / L, log-sum-exp, strided store ----
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l = sum_xor32(lsum[rb]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (p.lse != nullptr && hh == 0 && qrow[rb] < p.q_len)
      p.lse[b * p.lse_sb + h * p.lse_sh + qrow[rb]] =
          l > 0.0f ? (mref[rb] + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : kNegInf;
    if (qrow[rb] < p.q_len) {
      OutT* orow = og + (int64_t)qrow[rb] * p.o_ss;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * db + 8 * g + 4 * hh;
          store4<OutT>(orow + col, oacc[rb][db][4 * g] * inv, oacc[rb][db][4 * g + 1] * inv,
                       oacc[rb][db][4 * g + 2] * inv, oacc[rb][db][4 * g + 3] * inv);
        }
    }
  }
}

template <int QB, typename OutT>
hipError_t launch_rows64(const FwdParams& p, hipStream_t stream) {
  const int64_t nitems = QB == 2 ? (p.nq + 1) / 2 : p.nq;
  const int64_t total = nitems * p.B * p.H;
  if (total == 0) return hipSuccess;
  const int64_t per_xcd = (total + 7) / 8;
  // units per group on an XCD, as in the forward (K/V of the group's heads
  // within about half of the last-level cache)
  int grouped = 0;
  const int units = p.B * p.kv_heads;
  if (units % 8 == 0) {
    const double kv_unit = 4.0 * p.kv_len * p.head_dim;
    grouped = 1;
    while (grouped < 8 && 2 * grouped <= units / 8 && 2 * grouped * kv_unit <= 16.0 * 1024 * 1024) grouped *= 2;
  }
  hipLaunchKernelGGL((splash_fwd_rows64_kernel<QB, OutT>), dim3((unsigned)(per_xcd * 8)), dim3(256), 0, stream, p,
                     (int)total, (int)per_xcd, grouped);
  return hipGetLastError();
}

template <typename OutT>
hipError_t launch_rows64_bq(const FwdParams& p, hipStream_t stream) {
  if (p.block_q == 128) return launch_rows64<2, OutT>(p, stream);
  return launch_rows64<1, OutT>(p, stream);  // block_q 256
}

}  // namespace

bool fwd_rows64_applies(const FwdParams& p, bool pointwise) {
  // softmax, D = 128, the band as the only element mask (segment ids and
  // dense masks take the one-block kernel), block_q 128 or 256
  if (pointwise || p.head_dim != 128 || p.mask_blocks != nullptr || p.q_seg != nullptr) return false;
  if (p.block_q != 128 && p.block_q != 256) return false;
  // SPLASH_FWD_ROWS64=1 or 0 in the environment picks this kernel or the
  // one-block one for every call it applies to (both compute the same
  // function; tests run both)
  const char* force = std::getenv("SPLASH_FWD_ROWS64");
  if (force != nullptr && (force[0] == '0' || force[0] == '1')) return force[0] == '1';
  // by default, at least four 256-row workgroups per slot (two per CU): with
  // fewer, the one-block kernel's smaller workgroups balance the tail better
  // (B=4 H=16 S=2048: 0.093 ms against 0.112 with 512 of these workgroups)
  const int64_t items = (int64_t)(p.block_q == 128 ? (p.nq + 1) / 2 : p.nq) * p.B * p.H;
  return items >= 4 * 512;
}

hipError_t launch_fwd_rows64(const FwdParams& p, bool out_f32, hipStream_t stream) {
  return out_f32 ? launch_rows64_bq<float>(p, stream) : launch_rows64_bq<__bf16>(p, stream);
}

}  // namespace splash
