// Attention backward (pointwise SiLU and softmax), bf16 inputs, CDNA4 matrix cores.
//
// What is computed ("hstu_ops.py" (RecML), _pointwise_splash_attention_bwd_kernel_impl):
// with x = scale q·k, sig = logistic(x) (0 where the mask forbids the pair),
//   p  = x sig / q_len                      dV_k += sum_q p dO_q
//   dp = dO_q · v_k
//   ds = dp sig (1 + x (1 - sig)) / q_len   dK_k += scale sum_q ds q_q
//                                           dQ_q += scale sum_k ds k_k
// Here the weights are kept without the constant factors (p' = t sig with
// t = -scale log2(e) q·k, ds' = dp (sig + x sig (1 - sig)), the same as
// dp sig (1 + x (1 - sig))); the factors -ln 2 / q_len (dV) and scale / q_len
// (dK, dQ) are applied once to each sum.
//
// Two kernels, each with its own walk over the non-empty blocks, neither
// needing any cross-workgroup reduction:
//   * dK / dV: one workgroup per (b, K/V head, kv block j), wavefront w owning
//     keys j bkv + 32 w .. + 31. The kv block's column is walked over q
//     blocks with the column metadata (data_next along q blocks, as the
//     page's dK/dV grid walks q steps with _next_nonzero(next_i=True)),
//     for every query head that reads this K/V head. Q and dO come through
//     LDS in tiles of 32 queries (direct HBM -> LDS copies, double-buffered);
//     the wavefront's K and V rows stay in registers as B operands:
//       S  = Q Kᵀ,  dP = dO Vᵀ        (A = Q / dO rows from LDS)
//       dVᵀ += dOᵀ P',  dKᵀ += Qᵀ dS'  (A = transposing LDS reads of dO / Q)
//     so the probabilities go from the accumulator straight into the B
//     operand, as in the forward.
//   * dQ: one workgroup per (b, query head, q block i), the forward's row walk
//     with Q and dO in registers: Sᵀ = K Qᵀ, dPᵀ = V dOᵀ, dQᵀ += Kᵀ dSᵀ.
// The dK/dV pass recomputes S and dP that the dQ pass also forms (7 products
// per block pair instead of 5), in exchange for deterministic sums with no
// atomics and no per-kv-block partial dQ.
//
// Softmax attention (SM) runs through the same two kernels with the softmax
// derivative instead (the gradient of page 3 section 12's definition, given
// the forward's per-row log-sum-exp LSE and delta = rowsum(dO * O)):
//   P = e^(x - LSE) (0 where masked), dV += Pᵀ dO, dS = P (dP - delta),
//   dK += scale dSᵀ Q, dQ += scale dS K.
// The dK/dV kernel copies the tile's LSE and delta values to LDS beside the
// Q and dO tiles; the dQ kernel keeps its query's two values in registers.

#include <type_traits>

#include "cdna4.h"

namespace splash {
namespace {

// Weights of one score from t = nl q·k (nl = -scale log2(e), so that
// 2^t = e^-x with x = scale q·k = -t ln 2): sig = 1 / (1 + 2^t),
// p = t sig (= -x sig / ln 2: the factor -ln 2 goes into dV's final factor)
// and ds' = dp (sig + x sig (1 - sig)) = dp (sig + p (sig - 1) ln 2), that
// last factor formed with two fmas. A masked score is given t = kMaskedT:
// 2^t overflows, sig = 0 and p = ds' = 0 through the same arithmetic (any
// t > 128 does the same, so large real exponents are safe too).
struct Weights {
  float p, ds;
};
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaskedT = 256.0f;
__device__ inline Weights pointwise_weights(float t, float dp) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
  const float pt = t * sg;
  const float w = __builtin_fmaf(sg, kLn2, -kLn2);  // (sig - 1) ln 2
  return {pt, dp * __builtin_fmaf(pt, w, sg)};
}

// XCD-aware work order shared by both passes: workgroup ids are dealt
// round-robin to the 8 XCDs. When the number of units is a multiple of 8, XCD
// x takes units x, x + 8, ... in groups of `units_grouped` units, and within a
// group the work items go heaviest first across all the group's units (a
// unit's items are listed heaviest first, `inner` consecutive items at a time
// being of equal weight); else (units_grouped = 0) each XCD takes a
// contiguous eighth of the work list. Returns false for an id past the end.
__device__ inline bool work_item(int per_unit, int inner, int total_work, int work_per_xcd, int units_grouped,
                                 int& unit, int& rest) {
  const int xcd = (int)(blockIdx.x & 7), k_in_xcd = (int)(blockIdx.x >> 3);
  if (units_grouped) {
    const int G = units_grouped;
    const int units_xcd = total_work / (8 * per_unit);
    const int gi = k_in_xcd / (G * per_unit);
    const int g_units = units_xcd - gi * G < G ? units_xcd - gi * G : G;  // the last group may be smaller
    const int r = k_in_xcd - gi * G * per_unit;
    const int rank = r / (g_units * inner);
    const int rem = r - rank * g_units * inner;
    const int ug = rem / inner;
    unit = xcd + 8 * (gi * G + ug);
    rest = rank * inner + (rem - ug * inner);
    return true;
  }
  const int wid = xcd * work_per_xcd + k_in_xcd;
  if (wid >= total_work) return false;
  unit = wid / per_unit;
  rest = wid - unit * per_unit;
  return true;
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------

template <int D, int NW>
struct DkvTiling {
  static constexpr int QC = 32;                  // queries per LDS tile
  static constexpr int ROWB = D * 2;
  static constexpr int RPI = 64 / (D / 8);       // rows per direct-copy instruction
  static constexpr int TILE = QC * ROWB;
  static constexpr int LOADS = (QC / RPI) / NW;  // copies per wave per matrix per tile
  static constexpr int SEG_ROWS = QC / NW;       // query ids copied per wave per tile
  static constexpr int NS = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int SEG_OFF = 2 * 2 * TILE;   // [stage][Q | dO][TILE], then [stage][QC] ids
  static constexpr int STAT_OFF = SEG_OFF + 2 * QC * 4;  // softmax: [stage][LSE | delta][QC] floats
  // dense masks: [stage][NW key words][QC query rows] words of the block's entry
  static constexpr int DM_WORDS = NW * QC;
  static constexpr int DM_OFF = STAT_OFF + 2 * 2 * QC * 4;
  static constexpr int LDS_BYTES = DM_OFF + 2 * DM_WORDS * 4;
  static_assert(LOADS >= 1, "tile too small for the workgroup");
};

// D = 64: about 170 VGPRs, two wavefronts per SIMD. D = 128: K, V and the
// two accumulators alone take 192 VGPRs, and the whole step about 270, more
// than two wavefronts per SIMD can hold without spilling, so D = 128 runs the
// paired kernel below instead (the value here only keeps the template whole).
template <int D>
constexpr int dkv_waves() {
  return D == 64 ? 2 : 1;
}

template <int D, int NW, bool SM, typename OutT, int MK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(dkv_waves<D>(), dkv_waves<D>())))
void bwd_dkv_bf16_kernel(BwdParams p, int total_work, int work_per_xcd, int units_grouped) {
  using T = DkvTiling<D, NW>;
  constexpr int NS = T::NS;
  constexpr int ND = T::ND;
  constexpr int QC = T::QC;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  int unit, j;
  if (!work_item(p.c_nk, 1, total_work, work_per_xcd, units_grouped, unit, j)) return;
  // j ascending: under causal masks the first kv blocks have the longest columns
  const int b = unit / p.kv_heads;
  const int hk = unit - b * p.kv_heads;
  const int bm = p.meta_batch == 1 ? 0 : b;
  const int G = p.kv_group;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int key = j * p.c_block_kv + wave * 32 + l32;
  const bool kvalid = key < p.kv_len;
  const bool has_seg = MK == kAnyMask ? p.q_seg != nullptr : MK == kSegments;

  // ---- this lane's key: K and V rows as B operands (head-dim 16 s + 8 hh ..) ----
  bf16x8 kreg[NS], vreg[NS];
  {
    const __bf16* kr = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + hk * p.k_sh + (int64_t)key * p.k_ss;
    const __bf16* vr = reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + hk * p.v_sh + (int64_t)key * p.v_ss;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      i16x8 a = {0, 0, 0, 0, 0, 0, 0, 0}, c = {0, 0, 0, 0, 0, 0, 0, 0};
      if (kvalid) {
        a = *reinterpret_cast<const i16x8*>(kr + 16 * s + 8 * hh);
        c = *reinterpret_cast<const i16x8*>(vr + 16 * s + 8 * hh);
      }
      kreg[s] = __builtin_bit_cast(bf16x8, a);
      vreg[s] = __builtin_bit_cast(bf16x8, c);
    }
  }
  const int32_t kseg = (has_seg && kvalid) ? p.kv_seg[(int64_t)b * p.kv_len + key] : 0;

  int aoff[NS];
  row_operand_offsets<D>(lane, aoff);
  int toff[2][ND];
  transpose_operand_offsets<D>(lane, toff);
  const uint32_t q_rs = (uint32_t)(p.q_ss * 2), do_rs = (uint32_t)(p.do_ss * 2);
  uint32_t qsel[T::LOADS], dsel[T::LOADS];
  tile_copy_offsets<D, NW>(lane, wave, q_rs, qsel);
  tile_copy_offsets<D, NW>(lane, wave, do_rs, dsel);
  const int32_t* qseg_b = p.q_seg + (int64_t)b * p.q_len;

  // ---- column walk over (query head of the group, q block, 32-query tile) ----
  // Walk state of one query head: its Q, dO and statistics rows and its
  // metadata column (stored by columns: c_nq consecutive entries), for the
  // head of the most recently issued tile. The parameters it is made from
  // are read from the kernarg segment on a head change only, which keeps
  // them out of the loop's scalar registers.
  const char* q_h;
  const char* do_h;
  const float* lse_h;
  const float* delta_h;
  const int32_t* dn_col;
  const int8_t* cls_col;
  const int32_t* mn_col;  // dense masks: the column's mask_next entries
  auto set_head = [&](int g) {
    const auto* kp = kernarg_params<BwdParams>();
    const int h = hk * G + g;
    const int hm = kp->c_meta_heads == 1 ? 0 : h;
    const int64_t col = (((int64_t)bm * kp->c_meta_heads + hm) * kp->c_nk + j) * kp->c_nq;
    dn_col = kp->c_data_next + col;
    cls_col = kp->c_block_mask + col;
    mn_col = kp->c_mask_next + col;
    q_h = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(kp->q) + b * kp->q_sb + h * kp->q_sh);
    do_h = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(kp->d_o) + b * kp->do_sb + h * kp->do_sh);
    const int64_t st = b * kp->st_sb + h * kp->st_sh;
    lse_h = kp->lse + st;
    delta_h = kp->delta + st;
  };
  // data_next is only followed forward and within [0, nq], so any metadata
  // content ends the walk in bounds.
  auto first_i = [&]() {
    if (p.c_nq == 0) return p.c_nq;
    const int i = scalar_load_i32(dn_col);
    return (i >= 0 && i <= p.c_nq) ? i : p.c_nq;
  };
  auto next_i = [&](int i) {
    const int in = (i + 1 < p.c_nq) ? scalar_load_i32(dn_col + i + 1) : p.c_nq;
    return (in > i && in <= p.c_nq) ? in : p.c_nq;
  };
  // the first (g, i) at or after head g with a non-empty block (g == G: none)
  auto settle = [&](int& g, int& i) {
    while (i >= p.c_nq) {
      if (++g >= G) return;
      set_head(g);
      i = first_i();
    }
  };

  const bool dense = MK == kAnyMask ? p.c_mask_blocks != nullptr : MK == kDense;
  // Copy of tile (q block i, offset t): Q and dO rows, their ids and
  // statistics, and for a partial block of a dense mask the block's words of
  // these rows, stored by key word ([NW][QC]).
  auto issue_tile = [&](int stage, int i, int t, bool i_partial) {
    const int q0 = i * p.c_block_q + t;
    const int rows = p.q_len - q0 < QC ? p.q_len - q0 : QC;  // rows past the end read as 0
    char* qdst = smem + stage * 2 * T::TILE;
    char* ddst = qdst + T::TILE;
    const u32x4 qrs = buffer_rsrc(q_h + (int64_t)q0 * q_rs, (uint32_t)rows * q_rs);
    const u32x4 drs = buffer_rsrc(do_h + (int64_t)q0 * do_rs, (uint32_t)rows * do_rs);
    lds_copy_rows<T::LOADS, NW * 1024>(qrs, qsel, lds_addr(qdst + wave * T::RPI * T::ROWB));
    lds_copy_rows<T::LOADS, NW * 1024>(drs, dsel, lds_addr(ddst + wave * T::RPI * T::ROWB));
    if (dense && i_partial) {
      int m = scalar_load_i32(mn_col + i);
      m = m < 0 ? 0 : (m >= p.c_num_mask_blocks ? (int)p.c_num_mask_blocks - 1 : m);  // stays in the store
      const int wpr = p.c_block_kv / 32;  // = NW: the workgroup covers the whole kv block
      const u32x4 mrs =
          buffer_rsrc(p.c_mask_blocks + (int64_t)m * p.c_block_q * wpr, (uint32_t)(p.c_block_q * wpr * 4));
      const uint32_t* mdst = reinterpret_cast<const uint32_t*>(smem + T::DM_OFF) + stage * T::DM_WORDS;
      for (int e0 = wave * 64; e0 < T::DM_WORDS; e0 += NW * 64) {
        const int e = e0 + lane;  // key word e / QC, tile row e % QC
        if (e < T::DM_WORDS) lds_copy4(mrs, (uint32_t)(((t + e % QC) * wpr + e / QC) * 4), lds_addr(mdst + e0));
      }
    }
    if (has_seg) {
      const uint32_t sdst =
          lds_addr(reinterpret_cast<int32_t*>(smem + T::SEG_OFF) + stage * QC + wave * T::SEG_ROWS);
      const u32x4 srs = buffer_rsrc(qseg_b + q0, (uint32_t)(rows * 4));
      if (lane < T::SEG_ROWS) lds_copy4(srs, (uint32_t)((wave * T::SEG_ROWS + lane) * 4), sdst);
    }
    if constexpr (SM) {
      float* st = reinterpret_cast<float*>(smem + T::STAT_OFF) + stage * 2 * QC + wave * T::SEG_ROWS;
      const u32x4 lrs = buffer_rsrc(lse_h + q0, (uint32_t)(rows * 4));
      const u32x4 drs2 = buffer_rsrc(delta_h + q0, (uint32_t)(rows * 4));
      if (lane < T::SEG_ROWS) {
        lds_copy4(lrs, (uint32_t)((wave * T::SEG_ROWS + lane) * 4), lds_addr(st));
        lds_copy4(drs2, (uint32_t)((wave * T::SEG_ROWS + lane) * 4), lds_addr(st + QC));
      }
    }
  };

  // Zeroed tiles: rows a clipped copy leaves unwritten hold zeros, never NaN.
  for (int o = tid * 16; o < T::SEG_OFF; o += NW * 64 * 16)
    *reinterpret_cast<uint4*>(smem + o) = uint4{0u, 0u, 0u, 0u};
  __syncthreads();

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.0f;
      dv[db][r] = 0.0f;
    }
  const float nl = -p.scale * 1.4426950408889634f;
  const float cl = p.scale * 1.4426950408889634f;  // softmax: x log2(e) = cl q·k
  constexpr float kMasked = SM ? -__builtin_inff() : kMaskedT;

  int cur_g = 0, cur_t = 0;
  set_head(0);
  int cur_i = first_i();
  settle(cur_g, cur_i);
  if (cur_g < G) issue_tile(0, cur_i, 0, dense && block_class(cls_col, cur_i) == 1);

  auto step = [&](auto stage_tag) -> bool {
    constexpr int stage = decltype(stage_tag)::value;
    const bool partial = block_class(cls_col, cur_i) == 1;
    int ng = cur_g, ni = cur_i, nt = cur_t + QC;
    if (nt >= p.c_block_q || ni * p.c_block_q + nt >= p.q_len) {
      ni = next_i(ni);
      nt = 0;
      settle(ng, ni);
    }
    wait_vmcnt<0>();  // this wave's copies of the current tile are in LDS
    barrier_only();   // everyone's are, and the other stage is free again
    // raised issue priority while the wavefront forms S, dP and the weights;
    // back to normal for the dV/dK products
    __builtin_amdgcn_s_setprio(1);
    if (ng < G) issue_tile(stage ^ 1, ni, nt, dense && block_class(cls_col, ni) == 1);

    const int q0 = cur_i * p.c_block_q + cur_t;
    const char* qt = smem + stage * 2 * T::TILE;
    const char* dt = qt + T::TILE;
    const int32_t* sseg = reinterpret_cast<const int32_t*>(smem + T::SEG_OFF) + stage * QC;
    const float* sst = reinterpret_cast<const float*>(smem + T::STAT_OFF) + stage * 2 * QC;

    // ---- S = Q Kᵀ and dP = dO Vᵀ: 32 queries (rows) x this wave's 32 keys ----
    f32x16 sacc, pacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[r] = 0.0f;
      pacc[r] = 0.0f;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qt + aoff[s]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kreg[s], sacc, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(dt + aoff[s]);
      pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vreg[s], pacc, 0, 0, 0);
    }

    // element r: query q0 + 8 (r / 4) + 4 hh + r % 4, key `key`. On a partial
    // block the band, the sequence ends and (with ids) segment equality leave
    // the lane's key one run of queries [a, e] of the tile plus the id test;
    // full blocks take a path with no per-score test at all.
    // t: the exponent, in place (pointwise nl q·k; softmax (x - LSE) log2(e))
    f32x16& t = sacc;
    if constexpr (SM) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sst + 8 * u + 4 * hh);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) t[4 * u + v4] = __builtin_fmaf(sacc[4 * u + v4], cl, -kLog2e * l4[v4]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = sacc[r] * nl;
    }
    if (partial) {
      const auto* kp = kernarg_params<BwdParams>();
      const int bi = kp->band_heads == 1 ? 0 : hk * G + cur_g;
      const int band_lo = kp->band[bi].lo, band_hi = kp->band[bi].hi;
      int a = key - band_hi - q0;
      int e = key - band_lo - q0;
      a = a > 0 ? a : 0;
      e = e < p.q_len - 1 - q0 ? e : p.q_len - 1 - q0;
      e = e < QC - 1 ? e : QC - 1;
      if (e < a || !kvalid) a = e = QC;  // no query of the tile
      const uint32_t width = (uint32_t)(e - a);
      const int base = 4 * hh - a;
      if (dense) {
        // (dense-mask metadata is built with any segment ids folded in)
        const uint32_t* sdm = reinterpret_cast<const uint32_t*>(smem + T::DM_OFF) + stage * T::DM_WORDS + wave * QC;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 w4 = *reinterpret_cast<const uint4*>(sdm + 8 * u + 4 * hh);
          const uint32_t words[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const bool ok = ((uint32_t)(base + 8 * u + v4) <= width) & (bool)((words[v4] >> l32) & 1u);
            t[4 * u + v4] = ok ? t[4 * u + v4] : kMasked;
          }
        }
      } else if (has_seg) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int4 qs4 = *reinterpret_cast<const int4*>(sseg + 8 * u + 4 * hh);
          const int ids[4] = {qs4.x, qs4.y, qs4.z, qs4.w};
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int r = 4 * u + v4;
            const bool ok = ((uint32_t)(base + 8 * u + v4) <= width) & (ids[v4] == kseg);
            t[r] = ok ? t[r] : kMasked;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = ((uint32_t)(base + 8 * (r >> 2) + (r & 3)) <= width) ? t[r] : kMasked;
      }
    }
    bf16x8 pb[2], sb[2];
    if constexpr (SM) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sst + QC + 8 * u + 4 * hh);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int r = 4 * u + v4;
          const float pr = __builtin_amdgcn_exp2f(t[r]);
          pb[r >> 3][r & 7] = (__bf16)pr;
          sb[r >> 3][r & 7] = (__bf16)(pr * (pacc[r] - d4[v4]));
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const Weights w = pointwise_weights(t[r], pacc[r]);
        pb[r >> 3][r & 7] = (__bf16)w.p;
        sb[r >> 3][r & 7] = (__bf16)w.ds;
      }
    }

    __builtin_amdgcn_s_setprio(0);

    // ---- dVᵀ += dOᵀ P', dKᵀ += Qᵀ dS' over the 32 queries ----
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      const int rowbase = 16 * g2 * T::ROWB;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(dt + rowbase + toff[0][db]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(dt + rowbase + toff[1][db]));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[g2], dv[db], 0, 0, 0);
      }
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(qt + rowbase + toff[0][db]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(qt + rowbase + toff[1][db]));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[g2], dk[db], 0, 0, 0);
      }
    }

    cur_g = ng;
    cur_i = ni;
    cur_t = nt;
    return cur_g < G;
  };
  while (cur_g < G) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
  }

  // ---- pointwise: dK = (scale / q_len) dK', dV = (-ln 2 / q_len) dV';
  //      softmax:   dK = scale dK', dV = dV'; lane's key row ----
  if (kvalid) {
    const float ck = SM ? p.scale : p.scale * p.inv_q_len, cv = SM ? 1.0f : -kLn2 * p.inv_q_len;
    OutT* dkr = reinterpret_cast<OutT*>(p.dk) + b * p.dk_sb + hk * p.dk_sh + (int64_t)key * p.dk_ss;
    OutT* dvr = reinterpret_cast<OutT*>(p.dv) + b * p.dv_sb + hk * p.dv_sh + (int64_t)key * p.dv_ss;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * hh;
        store4<OutT>(dkr + col, dk[db][4 * g] * ck, dk[db][4 * g + 1] * ck, dk[db][4 * g + 2] * ck,
                     dk[db][4 * g + 3] * ck);
        store4<OutT>(dvr + col, dv[db][4 * g] * cv, dv[db][4 * g + 1] * cv, dv[db][4 * g + 2] * cv,
                     dv[db][4 * g + 3] * cv);
      }
  }
}

// ---------------------------------------------------------------------------
// dK / dV with paired wavefronts
// ---------------------------------------------------------------------------
//
// At D = 128 one wavefront holding K, V, dK and dV needs about 295 registers,
// so only one fits a SIMD. Here each 32-key group is split over two
// wavefronts:
//   role 0 holds K, forms S = Q Kᵀ, the weights (P for dV and the factor g
//          that turns dP into dS), and accumulates dVᵀ += dOᵀ P;
//   role 1 holds V, forms dP = dO Vᵀ, takes g from role 0 through LDS, forms
//          dS = dP g (pointwise) or g (dP - delta) (softmax, g = P), and
//          accumulates dKᵀ += Qᵀ dS.
// Same products as the single-wavefront kernel at about 200 registers per
// wavefront. A workgroup has NG key groups (2 NG wavefronts, 32 NG keys);
// kv blocks wider than that are split over several workgroups. With NG = 2
// two workgroups share a CU, and the roles of a workgroup's wavefront pairs
// swap with the parity of its id, so that each SIMD runs the exponentials of
// one role beside the matrix work of the other. A step takes 64 queries (two
// 32-query parts per wavefront), so the walk's per-step scalar work and the
// two workgroup barriers per step (the tile, then the exchange of g in bf16)
// are spread over twice the matrix work.

template <int D, int NG>
struct PairTiling {
  static constexpr int NW = 2 * NG;               // wavefronts
  static constexpr int KEYS = 32 * NG;            // keys per workgroup
  static constexpr int QC = 64;                   // queries per LDS tile (one step)
  static constexpr int PARTS = QC / 32;           // 32-query parts per step
  static constexpr int ROWB = D * 2;
  static constexpr int RPI = 64 / (D / 8);        // rows per direct-copy instruction
  static constexpr int TILE = QC * ROWB;
  static constexpr int CW = (QC / RPI) < NW ? (QC / RPI) : NW;  // wavefronts that copy tiles
  static constexpr int LOADS = (QC / RPI) / CW;   // copies per copying wave per matrix per tile
  static constexpr int SEG_ROWS = QC / NW;        // ids (and stats) copied per wave per tile
  static constexpr int NS = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int SEG_OFF = 2 * 2 * TILE;    // [stage][Q | dO][TILE], then [stage][QC] ids
  static constexpr int STAT_OFF = SEG_OFF + 2 * QC * 4;      // softmax: [stage][LSE | delta][QC]
  static constexpr int X_OFF = STAT_OFF + 2 * 2 * QC * 4;    // exchange: [NG][PARTS][2][64 lanes][16 B] bf16
  // dense masks: [stage][NG key words][QC query rows] words of the block's entry
  static constexpr int DM_WORDS = NG * QC;
  static constexpr int DM_OFF = X_OFF + NG * PARTS * 2048;
  static constexpr int LDS_BYTES = DM_OFF + 2 * DM_WORDS * 4;
  static_assert(LOADS >= 1 && SEG_ROWS >= 1, "tile too small for the workgroup");
};

template <int D, int NG, bool SM, typename OutT, int MK>
__global__ __launch_bounds__(2 * NG * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_pair_bf16_kernel(BwdParams p, int total_work, int work_per_xcd, int units_grouped) {
  using T = PairTiling<D, NG>;
  constexpr int NW = T::NW;
  constexpr int NS = T::NS;
  constexpr int ND = T::ND;
  constexpr int QC = T::QC;
  constexpr int PARTS = T::PARTS;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  const int sub = p.c_block_kv / T::KEYS;  // workgroups per kv block
  int unit, rest;
  if (!work_item(p.c_nk * sub, sub, total_work, work_per_xcd, units_grouped, unit, rest)) return;
  const int j = rest / sub;
  const int part_of_block = rest - j * sub;
  const int b = unit / p.kv_heads;
  const int hk = unit - b * p.kv_heads;
  const int bm = p.meta_batch == 1 ? 0 : b;
  const int G = p.kv_group;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // 0: S, P, dV; 1: dP, dS, dK (wave-uniform). With NG = 4 the pair (w, w + 4)
  // shares a SIMD; with NG = 2 the pairs alternate with the workgroup parity.
  const int role = NG == 4 ? wave / NG : ((wave / NG) ^ (int)(blockIdx.x & 1));
  const int kg = wave % NG;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int key = j * p.c_block_kv + part_of_block * T::KEYS + kg * 32 + l32;
  const bool kvalid = key < p.kv_len;
  const bool has_seg = MK == kAnyMask ? p.q_seg != nullptr : MK == kSegments;

  // ---- this lane's key row: K (role 0) or V (role 1) as the B operand ----
  bf16x8 breg[NS];
  {
    const __bf16* src = role == 0
        ? reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + hk * p.k_sh + (int64_t)key * p.k_ss
        : reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + hk * p.v_sh + (int64_t)key * p.v_ss;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      i16x8 a = {0, 0, 0, 0, 0, 0, 0, 0};
      if (kvalid) a = *reinterpret_cast<const i16x8*>(src + 16 * s + 8 * hh);
      breg[s] = __builtin_bit_cast(bf16x8, a);
    }
  }
  const int32_t kseg = (has_seg && kvalid) ? p.kv_seg[(int64_t)b * p.kv_len + key] : 0;

  // LDS offsets with the role's tile folded in: role 0 reads Q rows and dO
  // transposed, role 1 dO rows and Q transposed (dO sits TILE bytes after Q)
  int aoff[NS];
  row_operand_offsets<D>(lane, aoff);
  int toff[2][ND];
  transpose_operand_offsets<D>(lane, toff);
#pragma unroll
  for (int s = 0; s < NS; ++s) aoff[s] += role == 0 ? 0 : T::TILE;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int db = 0; db < ND; ++db) toff[hf][db] += role == 0 ? T::TILE : 0;
  const uint32_t q_rs = (uint32_t)(p.q_ss * 2), do_rs = (uint32_t)(p.do_ss * 2);
  uint32_t qsel[T::LOADS], dsel[T::LOADS];
  tile_copy_offsets<D, T::CW>(lane, wave, q_rs, qsel);
  tile_copy_offsets<D, T::CW>(lane, wave, do_rs, dsel);
  const int32_t* qseg_b = p.q_seg + (int64_t)b * p.q_len;

  // Walk state of one query head of the group: its Q, dO and statistics rows
  // and its metadata column (stored by columns: c_nq consecutive entries).
  // It always describes the head of the most recently issued tile.
  // (The parameters it is made from are read from the kernarg segment on a
  // head change only, which keeps them out of the loop's scalar registers.)
  const char* q_h;
  const char* do_h;
  const float* lse_h;
  const float* delta_h;
  const int32_t* dn_col;
  const int8_t* cls_col;
  const int32_t* mn_col;  // dense masks: the column's mask_next entries
  auto set_head = [&](int g) {
    const auto* kp = kernarg_params<BwdParams>();
    const int h = hk * G + g;
    const int hm = kp->c_meta_heads == 1 ? 0 : h;
    const int64_t col = (((int64_t)bm * kp->c_meta_heads + hm) * kp->c_nk + j) * kp->c_nq;
    dn_col = kp->c_data_next + col;
    cls_col = kp->c_block_mask + col;
    mn_col = kp->c_mask_next + col;
    q_h = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(kp->q) + b * kp->q_sb + h * kp->q_sh);
    do_h = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(kp->d_o) + b * kp->do_sb + h * kp->do_sh);
    const int64_t st = b * kp->st_sb + h * kp->st_sh;
    lse_h = kp->lse + st;
    delta_h = kp->delta + st;
  };
  auto first_i = [&]() {
    if (p.c_nq == 0) return p.c_nq;
    const int i = scalar_load_i32(dn_col);
    return (i >= 0 && i <= p.c_nq) ? i : p.c_nq;
  };
  auto next_i = [&](int i) {
    const int in = (i + 1 < p.c_nq) ? scalar_load_i32(dn_col + i + 1) : p.c_nq;
    return (in > i && in <= p.c_nq) ? in : p.c_nq;
  };
  auto settle = [&](int& g, int& i) {
    while (i >= p.c_nq) {
      if (++g >= G) return;
      set_head(g);
      i = first_i();
    }
  };

  const bool dense = MK == kAnyMask ? p.c_mask_blocks != nullptr : MK == kDense;
  auto issue_tile = [&](int stage, int i, int t, bool i_partial) {
    const int q0 = i * p.c_block_q + t;
    // rows past the end of the sequence or of the q block read as 0 (no contribution)
    int rows = p.q_len - q0 < QC ? p.q_len - q0 : QC;
    rows = p.c_block_q - t < rows ? p.c_block_q - t : rows;
    if (dense && i_partial) {
      // the block's words of these rows for the workgroup's NG key words,
      // stored by key word ([NG][QC]); rows past the block read as 0
      int m = scalar_load_i32(mn_col + i);
      m = m < 0 ? 0 : (m >= p.c_num_mask_blocks ? (int)p.c_num_mask_blocks - 1 : m);  // stays in the store
      const int wpr = p.c_block_kv / 32;
      const u32x4 mrs =
          buffer_rsrc(p.c_mask_blocks + (int64_t)m * p.c_block_q * wpr, (uint32_t)(p.c_block_q * wpr * 4));
      const uint32_t* mdst = reinterpret_cast<const uint32_t*>(smem + T::DM_OFF) + stage * T::DM_WORDS;
      for (int e0 = wave * 64; e0 < T::DM_WORDS; e0 += NW * 64) {
        const int e = e0 + lane;  // key word e / QC of the workgroup, tile row e % QC
        const uint32_t voff = (uint32_t)(((t + e % QC) * wpr + part_of_block * NG + e / QC) * 4);
        if (e < T::DM_WORDS) lds_copy4(mrs, voff, lds_addr(mdst + e0));
      }
    }
    if (wave < T::CW) {
      char* qdst = smem + stage * 2 * T::TILE;
      char* ddst = qdst + T::TILE;
      const u32x4 qrs = buffer_rsrc(q_h + (int64_t)q0 * q_rs, (uint32_t)rows * q_rs);
      const u32x4 drs = buffer_rsrc(do_h + (int64_t)q0 * do_rs, (uint32_t)rows * do_rs);
      lds_copy_rows<T::LOADS, T::CW * 1024>(qrs, qsel, lds_addr(qdst + wave * T::RPI * T::ROWB));
      lds_copy_rows<T::LOADS, T::CW * 1024>(drs, dsel, lds_addr(ddst + wave * T::RPI * T::ROWB));
    }
    if (has_seg) {
      const uint32_t sdst =
          lds_addr(reinterpret_cast<int32_t*>(smem + T::SEG_OFF) + stage * QC + wave * T::SEG_ROWS);
      const u32x4 srs = buffer_rsrc(qseg_b + q0, (uint32_t)(rows * 4));
      if (lane < T::SEG_ROWS) lds_copy4(srs, (uint32_t)((wave * T::SEG_ROWS + lane) * 4), sdst);
    }
    if constexpr (SM) {
      float* st = reinterpret_cast<float*>(smem + T::STAT_OFF) + stage * 2 * QC + wave * T::SEG_ROWS;
      const u32x4 lrs = buffer_rsrc(lse_h + q0, (uint32_t)(rows * 4));
      const u32x4 drs2 = buffer_rsrc(delta_h + q0, (uint32_t)(rows * 4));
      if (lane < T::SEG_ROWS) {
        lds_copy4(lrs, (uint32_t)((wave * T::SEG_ROWS + lane) * 4), lds_addr(st));
        lds_copy4(drs2, (uint32_t)((wave * T::SEG_ROWS + lane) * 4), lds_addr(st + QC));
      }
    }
  };

  for (int o = tid * 16; o < T::SEG_OFF; o += NW * 64 * 16)
    *reinterpret_cast<uint4*>(smem + o) = uint4{0u, 0u, 0u, 0u};
  __syncthreads();

  f32x16 acc[ND];  // role 0: dVᵀ, role 1: dKᵀ
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  const float nl = -p.scale * 1.4426950408889634f;
  const float cl = p.scale * 1.4426950408889634f;
  constexpr float kMasked = SM ? -__builtin_inff() : kMaskedT;
  // this lane's exchange slots: part u, chunk c at xg + (u * 2 + c) * 64
  bf16x8* xg = reinterpret_cast<bf16x8*>(smem + T::X_OFF + kg * PARTS * 2048) + lane;

  int cur_g = 0, cur_t = 0;
  set_head(0);
  int cur_i = first_i();
  settle(cur_g, cur_i);
  if (cur_g < G) issue_tile(0, cur_i, 0, dense && block_class(cls_col, cur_i) == 1);

  auto step = [&](auto stage_tag) -> bool {
    constexpr int stage = decltype(stage_tag)::value;
    const bool partial = block_class(cls_col, cur_i) == 1;
    int ng = cur_g, ni = cur_i, nt = cur_t + QC;
    if (nt >= p.c_block_q || ni * p.c_block_q + nt >= p.q_len) {
      ni = next_i(ni);
      nt = 0;
      settle(ng, ni);
    }
    __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<0>();  // this wave's copies of the current tile are in LDS
    barrier_only();   // everyone's are; the other stage and the exchange are free again
    if (ng < G) issue_tile(stage ^ 1, ni, nt, dense && block_class(cls_col, ni) == 1);

    const char* tb = smem + stage * 2 * T::TILE;  // Q tile, then dO tile
    const float* sst = reinterpret_cast<const float*>(smem + T::STAT_OFF) + stage * 2 * QC;

    // S = Q Kᵀ (role 0) or dP = dO Vᵀ (role 1): per part, 32 queries (rows) x 32 keys
    f32x16 c[PARTS];
#pragma unroll
    for (int u = 0; u < PARTS; ++u) {
#pragma unroll
      for (int r = 0; r < 16; ++r) c[u][r] = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(tb + 32 * u * T::ROWB + aoff[s]);
        c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, breg[s], c[u], 0, 0, 0);
      }
    }

    bf16x8 wb[PARTS][2];  // role 0: P, role 1: dS (B operands)
    if (role == 0) {
      const int q0 = cur_i * p.c_block_q + cur_t;
#pragma unroll
      for (int u = 0; u < PARTS; ++u) {
        // element r: query q0 + 32 u + 8 (r / 4) + 4 hh + r % 4, key `key`
        f32x16& t = c[u];
        if constexpr (SM) {
#pragma unroll
          for (int w4 = 0; w4 < 4; ++w4) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(sst + 32 * u + 8 * w4 + 4 * hh);
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) t[4 * w4 + v4] = __builtin_fmaf(t[4 * w4 + v4], cl, -kLog2e * l4[v4]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) t[r] = t[r] * nl;
        }
        if (partial) {
          const auto* kp = kernarg_params<BwdParams>();
          const int bi = kp->band_heads == 1 ? 0 : hk * G + cur_g;
          const int band_lo = kp->band[bi].lo, band_hi = kp->band[bi].hi;
          const int qp = q0 + 32 * u;
          int a = key - band_hi - qp;
          int e = key - band_lo - qp;
          a = a > 0 ? a : 0;
          e = e < p.q_len - 1 - qp ? e : p.q_len - 1 - qp;
          e = e < 31 ? e : 31;
          if (e < a || !kvalid) a = e = 32;
          const uint32_t width = (uint32_t)(e - a);
          const int base = 4 * hh - a;
          if (dense) {
            // (dense-mask metadata is built with any segment ids folded in)
            const uint32_t* sdm =
                reinterpret_cast<const uint32_t*>(smem + T::DM_OFF) + stage * T::DM_WORDS + kg * QC + 32 * u;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
              const uint4 ww = *reinterpret_cast<const uint4*>(sdm + 8 * w4 + 4 * hh);
              const uint32_t words[4] = {ww.x, ww.y, ww.z, ww.w};
#pragma unroll
              for (int v4 = 0; v4 < 4; ++v4) {
                const bool ok = ((uint32_t)(base + 8 * w4 + v4) <= width) & (bool)((words[v4] >> l32) & 1u);
                t[4 * w4 + v4] = ok ? t[4 * w4 + v4] : kMasked;
              }
            }
          } else if (has_seg) {
            const int32_t* sseg = reinterpret_cast<const int32_t*>(smem + T::SEG_OFF) + stage * QC + 32 * u;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
              const int4 qs4 = *reinterpret_cast<const int4*>(sseg + 8 * w4 + 4 * hh);
              const int ids[4] = {qs4.x, qs4.y, qs4.z, qs4.w};
#pragma unroll
              for (int v4 = 0; v4 < 4; ++v4) {
                const bool ok = ((uint32_t)(base + 8 * w4 + v4) <= width) & (ids[v4] == kseg);
                t[4 * w4 + v4] = ok ? t[4 * w4 + v4] : kMasked;
              }
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              t[r] = ((uint32_t)(base + 8 * (r >> 2) + (r & 3)) <= width) ? t[r] : kMasked;
          }
        }
        // P for dV, g for role 1 (bf16, through LDS)
        bf16x8 gp[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr, g;
          if constexpr (SM) {
            pr = __builtin_amdgcn_exp2f(t[r]);
            g = pr;
          } else {
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t[r]));
            pr = t[r] * sg;
            g = __builtin_fmaf(pr, __builtin_fmaf(sg, kLn2, -kLn2), sg);
          }
          wb[u][r >> 3][r & 7] = (__bf16)pr;
          gp[r >> 3][r & 7] = (__bf16)g;
        }
        xg[(2 * u) * 64] = gp[0];
        xg[(2 * u + 1) * 64] = gp[1];
      }
    }
    barrier_only();  // g of every key group is in LDS (the next tile's copies stay in flight)
    // role 1 (dS, then dK) issues at raised priority until the next tile
    // barrier, ahead of its role-0 partner on the SIMD (measured 1.8% faster
    // at s3h; raising role 0 before the exchange instead was not faster)
    if (role == 1) __builtin_amdgcn_s_setprio(1);
    if (role == 1) {
#pragma unroll
      for (int u = 0; u < PARTS; ++u) {
        const bf16x8 g0 = xg[(2 * u) * 64], g1 = xg[(2 * u + 1) * 64];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          f32x4 d4 = {0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (SM) d4 = *reinterpret_cast<const f32x4*>(sst + QC + 32 * u + 8 * w4 + 4 * hh);
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int r = 4 * w4 + v4;
            const float g = (float)(r < 8 ? g0[r] : g1[r - 8]);
            wb[u][r >> 3][r & 7] = (__bf16)(SM ? g * (c[u][r] - d4[v4]) : c[u][r] * g);
          }
        }
      }
    }

    // role 0: dVᵀ += dOᵀ P; role 1: dKᵀ += Qᵀ dS (toff carries the role's tile)
#pragma unroll
    for (int u = 0; u < PARTS; ++u)
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int rowbase = (32 * u + 16 * g2) * T::ROWB;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(tb + rowbase + toff[0][db]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(tb + rowbase + toff[1][db]));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wb[u][g2], acc[db], 0, 0, 0);
        }
      }

    cur_g = ng;
    cur_i = ni;
    cur_t = nt;
    return cur_g < G;
  };
  while (cur_g < G) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
  }

  // role 0 stores dV, role 1 dK (factors as in the single-wavefront kernel)
  if (kvalid) {
    const float cf = role == 0 ? (SM ? 1.0f : -kLn2 * p.inv_q_len) : (SM ? p.scale : p.scale * p.inv_q_len);
    OutT* dst = role == 0
        ? reinterpret_cast<OutT*>(p.dv) + b * p.dv_sb + hk * p.dv_sh + (int64_t)key * p.dv_ss
        : reinterpret_cast<OutT*>(p.dk) + b * p.dk_sb + hk * p.dk_sh + (int64_t)key * p.dk_ss;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * hh;
        store4<OutT>(dst + col, acc[db][4 * g] * cf, acc[db][4 * g + 1] * cf, acc[db][4 * g + 2] * cf,
                     acc[db][4 * g + 3] * cf);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

template <int D, int NW>
struct DqTiling {
  static constexpr int KC = D == 128 ? 32 : 64;  // keys per LDS tile
  static constexpr int ROWB = D * 2;
  static constexpr int RPI = 64 / (D / 8);
  static constexpr int TILE = KC * ROWB;
  static constexpr int LOADS = (KC / RPI) / NW;
  static constexpr int SEG_KEYS = KC / NW;
  static constexpr int NS = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int WPT = KC / 32;            // dense-mask words per query row per tile
  static constexpr int DM_WORDS = NW * 32 * WPT; // dense-mask words per tile (every row of the block)
  static constexpr int SEG_OFF = 2 * 2 * TILE;   // [stage][K | V][TILE], then [stage][KC] ids,
  static constexpr int DM_OFF = SEG_OFF + 2 * KC * 4;  // then [stage][DM_WORDS] dense-mask words
  static constexpr int LDS_BYTES = DM_OFF + 2 * DM_WORDS * 4;
  static_assert(LOADS >= 1, "tile too small for the workgroup");
};

// about 135 VGPRs at D = 64 and 215 at D = 128
template <int D>
constexpr int dq_waves() {
  return D == 64 ? 3 : 2;
}

template <int D, int NW, bool SM, typename OutT, int MK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(dq_waves<D>(), dq_waves<D>())))
void bwd_dq_bf16_kernel(BwdParams p, int total_work, int work_per_xcd, int units_grouped) {
  using T = DqTiling<D, NW>;
  constexpr int KC = T::KC;
  constexpr int NS = T::NS;
  constexpr int ND = T::ND;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  // unit = (b, K/V head) with its query heads; heaviest q blocks first
  int unit, rest;
  if (!work_item(p.nq * p.kv_group, p.kv_group, total_work, work_per_xcd, units_grouped, unit, rest)) return;
  const int ri = rest / p.kv_group;
  const int i = p.nq - 1 - ri;
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

  const char* kg = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + hk * p.k_sh);
  const char* vg = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + hk * p.v_sh);
  const int64_t k_rs = p.k_ss * 2, v_rs = p.v_ss * 2;
  const bool has_seg = MK == kAnyMask ? p.q_seg != nullptr : MK == kSegments;
  const int32_t* kvseg_g = has_seg ? p.kv_seg + (int64_t)b * p.kv_len : nullptr;

  // ---- this lane's query: Q and dO rows as B operands ----
  const int qrow = i * p.block_q + wave * 32 + l32;
  const bool qvalid = qrow < p.q_len;
  bf16x8 qreg[NS], oreg[NS];
  {
    const __bf16* qr = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)qrow * p.q_ss;
    const __bf16* orr = reinterpret_cast<const __bf16*>(p.d_o) + b * p.do_sb + h * p.do_sh + (int64_t)qrow * p.do_ss;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      i16x8 a = {0, 0, 0, 0, 0, 0, 0, 0}, c = {0, 0, 0, 0, 0, 0, 0, 0};
      if (qvalid) {
        a = *reinterpret_cast<const i16x8*>(qr + 16 * s + 8 * hh);
        c = *reinterpret_cast<const i16x8*>(orr + 16 * s + 8 * hh);
      }
      qreg[s] = __builtin_bit_cast(bf16x8, a);
      oreg[s] = __builtin_bit_cast(bf16x8, c);
    }
  }
  const int32_t myseg = (has_seg && qvalid) ? p.q_seg[(int64_t)b * p.q_len + qrow] : 0;
  // softmax: this query's LSE (log2 units) and delta
  float lse2 = 0.0f, dlt = 0.0f;
  if (SM && qvalid) {
    const int64_t off = b * p.st_sb + h * p.st_sh + qrow;
    lse2 = p.lse[off] * kLog2e;
    dlt = p.delta[off];
  }

  int aoff[NS];
  row_operand_offsets<D>(lane, aoff);
  int toff[2][ND];
  transpose_operand_offsets<D>(lane, toff);
  uint32_t ksel[T::LOADS], vsel[T::LOADS];
  tile_copy_offsets<D, NW>(lane, wave, k_rs, ksel);
  tile_copy_offsets<D, NW>(lane, wave, v_rs, vsel);

  const int64_t mrow = (((int64_t)bm * p.meta_heads + hm) * p.nq + i) * p.nk;
  const int8_t* bmask = p.block_mask + mrow;
  const int32_t* dnext = p.data_next + mrow;

  const bool dense = MK == kAnyMask ? p.mask_blocks != nullptr : MK == kDense;
  // Copy of tile (block jj, offset t): K and V rows, their segment ids, and
  // for a partial block of a dense mask the block's bits of this tile's keys.
  auto issue_tile = [&](int stage, int jj, int t, bool j_partial) {
    const int key0 = jj * p.block_kv + t;
    char* kdst = smem + stage * 2 * T::TILE;
    char* vdst = kdst + T::TILE;
    const int rows = p.kv_len - key0 < KC ? p.kv_len - key0 : KC;
    const u32x4 krs = buffer_rsrc(kg + key0 * k_rs, (uint32_t)(rows * k_rs));
    const u32x4 vrs = buffer_rsrc(vg + key0 * v_rs, (uint32_t)(rows * v_rs));
    lds_copy_rows<T::LOADS, NW * 1024>(krs, ksel, lds_addr(kdst + wave * T::RPI * T::ROWB));
    lds_copy_rows<T::LOADS, NW * 1024>(vrs, vsel, lds_addr(vdst + wave * T::RPI * T::ROWB));
    if (has_seg) {
      const uint32_t sdst = lds_addr(reinterpret_cast<int32_t*>(smem + T::SEG_OFF) + stage * KC + wave * T::SEG_KEYS);
      const u32x4 srs = buffer_rsrc(kvseg_g + key0, (uint32_t)(rows * 4));
      if (lane < T::SEG_KEYS) lds_copy4(srs, (uint32_t)((wave * T::SEG_KEYS + lane) * 4), sdst);
    }
    if (dense && j_partial) {
      int m = scalar_load_i32(p.mask_next + mrow + jj);
      m = m < 0 ? 0 : (m >= p.num_mask_blocks ? (int)p.num_mask_blocks - 1 : m);  // any content stays in the store
      const int wpr = p.block_kv / 32;
      const u32x4 drs = buffer_rsrc(p.mask_blocks + (int64_t)m * p.block_q * wpr, (uint32_t)(p.block_q * wpr * 4));
      const uint32_t* ddst = reinterpret_cast<const uint32_t*>(smem + T::DM_OFF) + stage * T::DM_WORDS;
      // word e of the tile: row e / WPT, word t / 32 + e % WPT of that row
      for (int e0 = wave * 64; e0 < T::DM_WORDS; e0 += NW * 64) {
        const int e = e0 + lane;
        const uint32_t voff = (uint32_t)(((e / T::WPT) * wpr + t / 32 + e % T::WPT) * 4);
        if (e < T::DM_WORDS) lds_copy4(drs, voff, lds_addr(ddst + e0));
      }
    }
  };

  for (int o = tid * 16; o < T::SEG_OFF; o += NW * 64 * 16)
    *reinterpret_cast<uint4*>(smem + o) = uint4{0u, 0u, 0u, 0u};
  __syncthreads();

  f32x16 dq[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.0f;
  const float nl = -p.scale * 1.4426950408889634f;
  const float cl = p.scale * 1.4426950408889634f;
  constexpr float kMasked = SM ? -__builtin_inff() : kMaskedT;

  auto next_block = [&](int jj) {
    const int jn = (jj + 1 < p.nk) ? scalar_load_i32(dnext + jj + 1) : p.nk;
    return (jn > jj && jn <= p.nk) ? jn : p.nk;
  };
  int cur_j = p.nk > 0 ? scalar_load_i32(dnext) : p.nk;
  if (cur_j < 0 || cur_j > p.nk) cur_j = p.nk;
  int cur_t = 0;
  // class of the block being walked, read once per block (off the tile's math)
  bool cur_partial = cur_j < p.nk && block_class(bmask, cur_j) == 1;
  if (cur_j < p.nk) issue_tile(0, cur_j, 0, cur_partial);

  auto step = [&](auto stage_tag) -> bool {
    constexpr int stage = decltype(stage_tag)::value;
    int nxt_j = cur_j, nxt_t = cur_t + KC;
    bool nxt_partial = cur_partial;
    if (nxt_t >= p.block_kv || cur_j * p.block_kv + nxt_t >= p.kv_len) {
      nxt_j = next_block(cur_j);
      nxt_t = 0;
      nxt_partial = nxt_j < p.nk && block_class(bmask, nxt_j) == 1;
    }
    wait_vmcnt<0>();
    barrier_only();
    if (nxt_j < p.nk) issue_tile(stage ^ 1, nxt_j, nxt_t, nxt_partial);
    // raised issue priority while the wavefront forms S, dP and dS (measured
    // faster at D = 64 and for the softmax gradient, slower for the pointwise
    // one at D = 128)
    constexpr bool kPrio = D == 64 || SM;
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);

    const int k0 = cur_j * p.block_kv + cur_t;
    const bool partial = cur_partial;
    const char* kt = smem + stage * 2 * T::TILE;
    const char* vt = kt + T::TILE;
    const int32_t* sseg = reinterpret_cast<const int32_t*>(smem + T::SEG_OFF) + stage * KC;
    const uint32_t* dmw = reinterpret_cast<const uint32_t*>(smem + T::DM_OFF) + stage * T::DM_WORDS +
                          (wave * 32 + l32) * T::WPT;  // this row's dense-mask words of the tile
#pragma unroll
    for (int kb = 0; kb < KC / 32; ++kb) {
      // ---- Sᵀ = K Qᵀ, dPᵀ = V dOᵀ: 32 keys (rows) x this wave's 32 queries ----
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.0f;
        pacc[r] = 0.0f;
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + kb * 32 * T::ROWB + aoff[s]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + kb * 32 * T::ROWB + aoff[s]);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, oreg[s], pacc, 0, 0, 0);
      }
      // element r: key k0 + 32 kb + 8 (r / 4) + 4 hh + r % 4, query qrow
      // t: the exponent, in place (pointwise nl q·k; softmax (x - LSE) log2(e))
      f32x16& t = sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = SM ? __builtin_fmaf(sacc[r], cl, -lse2) : sacc[r] * nl;
      if (partial) {
        int a = qrow + band.lo - k0;
        int e = qrow + band.hi - k0;
        a = a > 0 ? a : 0;
        e = e < p.kv_len - 1 - k0 ? e : p.kv_len - 1 - k0;
        e = e < KC - 1 ? e : KC - 1;
        if (e < a || !qvalid) a = e = KC;
        const uint32_t width = (uint32_t)(e - a);
        const int base = 4 * hh - a + 32 * kb;
        if (dense) {
          // (dense-mask metadata is built with any segment ids folded in)
          const uint32_t dbits = dmw[kb] >> (4 * hh);  // bit 8 (r / 4) + r % 4 for score r
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = ((uint32_t)(base + 8 * (r >> 2) + (r & 3)) <= width) &
                            (bool)((dbits >> (8 * (r >> 2) + (r & 3))) & 1u);
            t[r] = ok ? t[r] : kMasked;
          }
        } else if (has_seg) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int4 ks4 = *reinterpret_cast<const int4*>(sseg + 32 * kb + 8 * u + 4 * hh);
            const int ids[4] = {ks4.x, ks4.y, ks4.z, ks4.w};
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
              const int r = 4 * u + v4;
              const bool ok = ((uint32_t)(base + 8 * u + v4) <= width) & (ids[v4] == myseg);
              t[r] = ok ? t[r] : kMasked;
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) t[r] = ((uint32_t)(base + 8 * (r >> 2) + (r & 3)) <= width) ? t[r] : kMasked;
        }
      }
      bf16x8 sb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sb[r >> 3][r & 7] = SM ? (__bf16)(__builtin_amdgcn_exp2f(t[r]) * (pacc[r] - dlt))
                               : (__bf16)pointwise_weights(t[r], pacc[r]).ds;

      if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);

      // ---- dQᵀ += Kᵀ dSᵀ over these 32 keys ----
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int rowbase = (32 * kb + 16 * g2) * T::ROWB;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(kt + rowbase + toff[0][db]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(kt + rowbase + toff[1][db]));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[g2], dq[db], 0, 0, 0);
        }
      }
    }
    cur_j = nxt_j;
    cur_t = nxt_t;
    cur_partial = nxt_partial;
    return cur_j < p.nk;
  };
  while (cur_j < p.nk) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
  }

  if (qvalid) {
    const float cq = SM ? p.scale : p.scale * p.inv_q_len;
    OutT* dqr = reinterpret_cast<OutT*>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)qrow * p.dq_ss;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * hh;
        store4<OutT>(dqr + col, dq[db][4 * g] * cq, dq[db][4 * g + 1] * cq, dq[db][4 * g + 2] * cq,
                     dq[db][4 * g + 3] * cq);
      }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

struct Order {
  int64_t total, per_xcd;
  int grouped;
};
// Units: (b, K/V head); a grid of 8 * ceil(work / 8) ids. Units per group on
// an XCD: the largest power of two up to 8 whose streamed tiles (unit_bytes
// per unit), over all 8 XCDs at once, stay within about half of the 256 MB
// last-level cache, as in the forward.
Order order_for(int64_t units, int64_t per_unit, double unit_bytes) {
  const int64_t total = units * per_unit;
  int g = 0;
  if (units % 8 == 0) {
    g = 1;
    while (g < 8 && 2 * g <= units / 8 && 2 * g * unit_bytes <= 16.0 * 1024 * 1024) g *= 2;
  }
  return {total, (total + 7) / 8, g};
}

template <int D, int NW, bool SM, typename OutT, int MK>
hipError_t launch_dkv(const BwdParams& p, hipStream_t stream) {
  // a dK/dV unit streams Q and dO of its kv_group query heads
  const Order o = order_for((int64_t)p.B * p.kv_heads, p.c_nk, 4.0 * p.q_len * p.head_dim * p.kv_group);
  if (o.total == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkv_bf16_kernel<D, NW, SM, OutT, MK>), dim3((unsigned)(o.per_xcd * 8)), dim3(NW * 64), 0,
                     stream, p, (int)o.total, (int)o.per_xcd, o.grouped);
  return hipGetLastError();
}

template <int D, int NW, bool SM, typename OutT, int MK>
hipError_t launch_dq(const BwdParams& p, hipStream_t stream) {
  // a dQ unit streams K and V of its K/V head
  const Order o = order_for((int64_t)p.B * p.kv_heads, (int64_t)p.nq * p.kv_group, 4.0 * p.kv_len * p.head_dim);
  if (o.total == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, NW, SM, OutT, MK>), dim3((unsigned)(o.per_xcd * 8)), dim3(NW * 64), 0,
                     stream, p, (int)o.total, (int)o.per_xcd, o.grouped);
  return hipGetLastError();
}

template <int D, int NG, bool SM, typename OutT, int MK>
hipError_t launch_dkv_pair(const BwdParams& p, hipStream_t stream) {
  const Order o = order_for((int64_t)p.B * p.kv_heads, (int64_t)p.c_nk * (p.c_block_kv / (32 * NG)),
                            4.0 * p.q_len * p.head_dim * p.kv_group);
  if (o.total == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkv_pair_bf16_kernel<D, NG, SM, OutT, MK>), dim3((unsigned)(o.per_xcd * 8)), dim3(2 * NG * 64),
                     0, stream, p, (int)o.total, (int)o.per_xcd, o.grouped);
  return hipGetLastError();
}

// The element-mask kind of each walk's instance: its own dense-mask store,
// else segment ids, else the band alone.
inline int dkv_mask_kind(const BwdParams& p) {
  return p.c_mask_blocks != nullptr ? kDense : (p.q_seg != nullptr ? kSegments : kBandOnly);
}
inline int dq_mask_kind(const BwdParams& p) {
  return p.mask_blocks != nullptr ? kDense : (p.q_seg != nullptr ? kSegments : kBandOnly);
}

template <int D, bool SM, typename OutT, int MK>
hipError_t launch_dkv_mk(const BwdParams& p, hipStream_t stream) {
  if constexpr (D == 128) {
    // paired wavefronts: K, V, dK and dV do not fit one wavefront twice per
    // SIMD. 128-key blocks: one eight-wavefront workgroup per CU (each tile
    // copy serves 128 keys, and a SIMD's two wavefronts work in step);
    // 64-key blocks: two four-wavefront workgroups per CU.
    return p.c_block_kv % 128 == 0 ? launch_dkv_pair<D, 4, SM, OutT, MK>(p, stream)
                                   : launch_dkv_pair<D, 2, SM, OutT, MK>(p, stream);
  } else {
    return p.c_block_kv == 64 ? launch_dkv<D, 2, SM, OutT, MK>(p, stream) : launch_dkv<D, 4, SM, OutT, MK>(p, stream);
  }
}

template <int D, bool SM, typename OutT, int MK>
hipError_t launch_dq_mk(const BwdParams& p, hipStream_t stream) {
  if (p.block_q == 64) return launch_dq<D, 2, SM, OutT, MK>(p, stream);
  if (p.block_q == 256) return launch_dq<D, 8, SM, OutT, MK>(p, stream);
  return launch_dq<D, 4, SM, OutT, MK>(p, stream);
}

template <int D, bool SM, typename OutT>
hipError_t launch_sm(const BwdParams& p, hipStream_t stream) {
  if constexpr (D == 64) {
    // One instance for every kind of mask at D = 64: the band-only instances
    // measured slower there (pointwise 8 x 8 x 4096 x 64: dK/dV 355 -> 369 us,
    // dQ 266 -> 269 us), while at D = 128 they shed the scalar spills of the
    // paired dK/dV kernel (softmax 2 x 32 x 8192 x 128: 4.05 -> 3.77 ms).
    const hipError_t e = launch_dkv_mk<D, SM, OutT, kAnyMask>(p, stream);
    if (e != hipSuccess) return e;
    return launch_dq_mk<D, SM, OutT, kAnyMask>(p, stream);
  } else {
    const int kd = dkv_mask_kind(p);
    const hipError_t e = kd == kDense      ? launch_dkv_mk<D, SM, OutT, kDense>(p, stream)
                         : kd == kSegments ? launch_dkv_mk<D, SM, OutT, kSegments>(p, stream)
                                           : launch_dkv_mk<D, SM, OutT, kBandOnly>(p, stream);
    if (e != hipSuccess) return e;
    const int kq = dq_mask_kind(p);
    return kq == kDense      ? launch_dq_mk<D, SM, OutT, kDense>(p, stream)
           : kq == kSegments ? launch_dq_mk<D, SM, OutT, kSegments>(p, stream)
                             : launch_dq_mk<D, SM, OutT, kBandOnly>(p, stream);
  }
}

template <int D, typename OutT>
hipError_t launch_d(const BwdParams& p, hipStream_t stream) {
  return p.softmax ? launch_sm<D, true, OutT>(p, stream) : launch_sm<D, false, OutT>(p, stream);
}

}  // namespace

hipError_t launch_pointwise_bwd_bf16(const BwdParams& p, bool out_f32, hipStream_t stream) {
  if (p.head_dim == 64) return out_f32 ? launch_d<64, float>(p, stream) : launch_d<64, __bf16>(p, stream);
  return out_f32 ? launch_d<128, float>(p, stream) : launch_d<128, __bf16>(p, stream);
}

}  // namespace splash
