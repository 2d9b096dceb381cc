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
// Work decomposition: one workgroup per (b, h, q block) with NW = block_q / 32
// wavefronts; each wavefront owns 32 query rows. The kv axis is walked in
// tiles of KC keys (32 or 64): K and V tiles are copied HBM -> LDS by direct (VGPR-free)
// 16-byte-per-lane loads, double-buffered so the copy of tile t+1 runs under
// the math of tile t.
//
// Matrix-core layout: scores are formed transposed, Sᵀ = K Qᵀ, with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Qᵀ held in registers for
// the whole kernel). In the 32x32 accumulator layout lane l holds column
// l % 32 (its query row) and 16 rows (keys), so row max / row sum are
// in-lane reductions plus one exchange between the half-waves, and the
// probabilities already sit in the B-operand layout of Oᵀ += Vᵀ Pᵀ: P never
// leaves registers. Vᵀ is read from the row-major V tile with the gfx950
// transposing LDS read (ds_read_b64_tr_b16), in the key order the
// accumulator gives P.
//
// LDS tiles are row-major (one key per row, head_dim contiguous) with the
// 16-byte chunks of row r stored at a row-dependent XOR-swizzled position
// (swz below), which keeps the K operand reads and the transposing V reads
// free of bank conflicts; the direct loads write that layout by choosing which
// global chunk each lane fetches.
//
// Softmax bookkeeping is in the log2 domain with the scale folded into one
// FMA before exp2, against a per-row reference m that O and L always share
// (so the result is the plain softmax whatever m is). Probabilities are first
// formed on the current m without computing a max; only when their sum shows
// a score more than 40 log2 units above m (or the row has no m yet) is the
// 32-key max taken and m raised, if that max exceeds m by more than 32, with
// O and L rescaled. Probabilities thus stay below 2^40, far from the
// fp32/bf16 range limit, and the max is computed about once per row.
//
// Pointwise: P = s sigmoid(c s) with the constant c / q_len applied to O once
// at the end.

#include <type_traits>

#include "cdna4.h"

namespace splash {
namespace {

constexpr float kRescaleSlack = 32.0f;  // log2 units a tile max may exceed the reference by
// A lane's sum of 16 probabilities above this means some score rose over 40
// log2 units above the reference (and a NaN or inf sum fails the test too).
constexpr float kFastLimit = 1099511627776.0f;  // 2^40

// Keys per LDS tile: 32 at D = 128 for up to four wavefronts (the smaller
// tiles let three workgroups share a CU's LDS, so three wavefronts share each
// SIMD), else 64.
template <int D, int NW>
constexpr int tile_keys() {
  return (D == 128 && NW <= 4) ? 32 : 64;
}
// Wavefronts per SIMD the register budget is set for.
template <int D, int NW>
constexpr int waves_per_simd() {
  return D == 64 ? 4 : (NW <= 4 ? 3 : 2);
}

template <int D, int NW>
struct Tiling {
  static constexpr int KC = tile_keys<D, NW>();
  static constexpr int NT = NW * 64;            // threads
  static constexpr int ROWB = D * 2;            // bytes per key row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows written by one direct-load instruction
  static constexpr int TILE = KC * ROWB;        // bytes of one K or V tile
  static constexpr int LOADS = (KC / RPI) / NW; // direct loads per wave per matrix per tile
  static constexpr int SEG_KEYS = KC / NW;      // segment ids loaded per wave per tile
  static constexpr int NS = D / 16;             // k-steps of the QKᵀ contraction
  static constexpr int ND = D / 32;             // 32-wide output blocks
  static constexpr int WPT = KC / 32;           // dense-mask words per query row per tile
  static constexpr int DM_WORDS = NW * 32 * WPT; // dense-mask words per tile (every row of the block)
  // LDS: [stage][K | V][TILE], [stage][KC] int32 segment ids, [stage][DM_WORDS]
  // dense-mask words
  static constexpr int SEG_OFF = 2 * 2 * TILE;
  static constexpr int DM_OFF = SEG_OFF + 2 * KC * 4;
  static constexpr int LDS_BYTES = DM_OFF + 2 * DM_WORDS * 4;
};

// Wavefronts per SIMD: at D = 128 a wavefront needs up to 168 VGPRs, so
// three (two for 8-wavefront workgroups, whose LDS allows only one per CU);
// at D = 64 four fit, and the extra wavefronts hide the longer vector work
// (per key, the pointwise variant spends two transcendentals on half as many
// matrix FLOPs).
template <int D, int NW, bool PW, typename OutT, int MK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(waves_per_simd<D, NW>(),
                                                                      waves_per_simd<D, NW>())))
void splash_fwd_bf16_kernel(FwdParams p, int total_work, int work_per_xcd, int units_grouped) {
  constexpr bool has_seg = MK == kSegments;
  constexpr bool dense = MK == kDense;
  using T = Tiling<D, NW>;
  constexpr int KC = T::KC;
  constexpr int NS = T::NS;
  constexpr int ND = T::ND;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  // XCD-aware order: workgroup ids are dealt round-robin to the 8 XCDs, so
  // id -> (x, k) = (id % 8, id / 8) is the k-th workgroup XCD x runs. A unit
  // is a K/V head together with the kv_group query heads that read it (one
  // head without grouping). When the number of units is a multiple of 8, XCD
  // x takes units x, x + 8, ... (units with different masks, say causal and
  // local heads, are then spread evenly over the XCDs), in groups of
  // `units_grouped` units: within a group the query blocks go heaviest first
  // (most kv blocks under causal masks) across all the group's units and
  // heads, so the group's tail is made of its lightest blocks, while the
  // K/V heads in flight stay few enough to be served from cache. Otherwise
  // (units_grouped = 0) each XCD takes a contiguous eighth of the work list.
  const int xcd = (int)(blockIdx.x & 7), k_in_xcd = (int)(blockIdx.x >> 3);
  const int per_unit = p.nq * p.kv_group;
  int unit, rest;
  if (units_grouped) {
    const int G = units_grouped;
    const int units_xcd = (p.B * p.kv_heads) / 8;
    const int gi = k_in_xcd / (G * per_unit);
    const int g_units = units_xcd - gi * G < G ? units_xcd - gi * G : G;  // the last group may be smaller
    const int r = k_in_xcd - gi * G * per_unit;
    const int ri0 = r / (g_units * p.kv_group);  // rank of the query block, heaviest first
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
  const int i = p.nq - 1 - ri;
  const int b = unit / p.kv_heads;
  const int hk = unit - b * p.kv_heads;  // K/V head
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
  const int64_t k_rs = p.k_ss * 2;  // bytes between key rows
  const int64_t v_rs = p.v_ss * 2;
  const int32_t* kvseg_g = has_seg ? p.kv_seg + (int64_t)b * p.kv_len : nullptr;

  // ---- Q (B operand of Sᵀ = K Qᵀ), two 32-row column blocks per wave ----
  // Softmax only depends on scale through scale * scores; a negative scale is
  // applied as an exact sign flip of Q so the fused exponent uses c >= 0.
  const bool negate_q = !PW && p.scale < 0.0f;
  // (a zero scale is taken as the smallest normal float: every allowed score
  // then gets the same weight, and -inf * c stays -inf for masked ones)
  const float c = PW ? p.scale : fmaxf(negate_q ? -p.scale_log2 : p.scale_log2, 1.17549435e-38f);
  const int qrow = i * (NW * 32) + wave * 32 + l32;
  bf16x8 qreg[NS];
  int32_t myseg = 0;
  {
    // rows past the end read the last row (no branch around the loads, so
    // they all issue at once) and are then zeroed
    const bool valid = qrow < p.q_len;
    const __bf16* qrow_ptr = qg + (int64_t)(valid ? qrow : p.q_len - 1) * p.q_ss + 8 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      i16x8 v = *reinterpret_cast<const i16x8*>(qrow_ptr + 16 * s);
      if (negate_q) v ^= (short)0x8000;
      if (!valid) v = (i16x8){0, 0, 0, 0, 0, 0, 0, 0};
      qreg[s] = __builtin_bit_cast(bf16x8, v);
    }
    if (has_seg && valid) myseg = p.q_seg[(int64_t)b * p.q_len + qrow];
  }

  // ---- per-lane LDS offsets (swizzled chunk positions) ----
  // K operand: rows 32 kb + l32 of the K tile; Vᵀ operand: transposing reads
  // of the V tile in the key order the accumulator gives P.
  int koff[NS];
  row_operand_offsets<D>(lane, koff);
  int voff[2][ND];
  transpose_operand_offsets<D>(lane, voff);

  // ---- direct HBM -> LDS copy of one K/V tile (plus segment ids) ----
  uint32_t kvsel[T::LOADS], vvsel[T::LOADS];
  tile_copy_offsets<D, NW>(lane, wave, k_rs, kvsel);
  tile_copy_offsets<D, NW>(lane, wave, v_rs, vvsel);
  const int64_t mrow = (((int64_t)bm * p.meta_heads + hm) * p.nq + i) * p.nk;
  const int8_t* bmask = p.block_mask + mrow;
  const int32_t* dnext = p.data_next + mrow;

  // Copy of tile (block j, offset t): K and V rows, their segment ids, and for
  // a partial block of a dense mask the block's bits of this tile's keys.
  auto issue_tile = [&](int stage, int j, int t, bool j_partial) {
    const int key0 = j * p.block_kv + t;
    char* kdst = smem + stage * 2 * T::TILE;
    char* vdst = kdst + T::TILE;
    const int rows = p.kv_len - key0 < KC ? p.kv_len - key0 : KC;  // rows past the end read as 0
    const u32x4 krs = buffer_rsrc(kg + key0 * k_rs, (uint32_t)(rows * k_rs));
    const u32x4 vrs = buffer_rsrc(vg + key0 * v_rs, (uint32_t)(rows * v_rs));
    lds_copy_rows<T::LOADS, NW * 1024>(krs, kvsel, lds_addr(kdst + wave * T::RPI * T::ROWB));
    lds_copy_rows<T::LOADS, NW * 1024>(vrs, vvsel, lds_addr(vdst + wave * T::RPI * T::ROWB));
    if constexpr (has_seg) {
      const uint32_t sdst = lds_addr(reinterpret_cast<int32_t*>(smem + T::SEG_OFF) + stage * KC + wave * T::SEG_KEYS);
      const u32x4 srs = buffer_rsrc(kvseg_g + key0, (uint32_t)(rows * 4));
      if (lane < T::SEG_KEYS) lds_copy4(srs, (uint32_t)((wave * T::SEG_KEYS + lane) * 4), sdst);
    }
    if constexpr (dense) if (j_partial) {
      int m = scalar_load_i32(p.mask_next + mrow + j);
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

  // The first non-empty kv block and its class, read ahead of the LDS set-up.
  int cur_j = p.nk > 0 ? scalar_load_i32(dnext) : p.nk;
  if (cur_j < 0 || cur_j > p.nk) cur_j = p.nk;
  int cur_t = 0;
  // class of the block being walked, read once per block (off the tile's math)
  bool cur_partial = cur_j < p.nk && block_class(bmask, cur_j) == 1;

  // The tiles start zeroed, so rows that a clipped copy leaves unwritten can
  // never hold NaN bit patterns (their probabilities are 0, and 0 * NaN is NaN).
  // (The barrier waits for the LDS stores only: the Q loads stay in flight
  // under the first tile copy.)
  for (int o = tid * 16; o < T::SEG_OFF; o += T::NT * 16)
    *reinterpret_cast<uint4*>(smem + o) = uint4{0u, 0u, 0u, 0u};
  barrier_only();

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float mref = kNegInf;  // reference max (log2 domain), shared by O and L
  float lsum = 0.0f;     // this lane's share of L


  // Walk: tiles of KC keys inside the non-empty blocks reached through
  // data_next. data_next is only followed forward and within [0, nk], so any
  // metadata content ends the walk in bounds.
  auto next_block = [&](int j) {
    const int jn = (j + 1 < p.nk) ? scalar_load_i32(dnext + j + 1) : p.nk;
    return (jn > j && jn <= p.nk) ? jn : p.nk;
  };
  if (cur_j < p.nk) issue_tile(0, cur_j, 0, cur_partial);

  // One tile in LDS stage STAGE (a compile-time constant, so every tile
  // address is a per-lane offset plus an immediate). Returns whether another
  // tile follows.
  auto step = [&](auto stage_tag) -> bool {
    constexpr int stage = decltype(stage_tag)::value;
    int nxt_j = cur_j, nxt_t = cur_t + KC;
    bool nxt_partial = cur_partial;
    if (nxt_t >= p.block_kv || cur_j * p.block_kv + nxt_t >= p.kv_len) {
      nxt_j = next_block(cur_j);
      nxt_t = 0;
      nxt_partial = nxt_j < p.nk && block_class(bmask, nxt_j) == 1;
    }
    wait_vmcnt<0>();  // this wave's copies of the current tile are in LDS
    // After this barrier every wave's copies of the current tile are in LDS and
    // every wave is done with the previous tile, whose stage is refilled now.
    barrier_only();
    // The wavefront issues at raised priority while it issues the next tile's
    // copies, reads K and forms S and the probabilities, and drops back before
    // P V: a wavefront entering its first matrix phase is then picked ahead of
    // the other wavefronts' work on the SIMD (measured faster than no raise,
    // or a raise in both matrix phases).
    __builtin_amdgcn_s_setprio(1);
    if (nxt_j < p.nk) issue_tile(stage ^ 1, nxt_j, nxt_t, nxt_partial);

    const int k0 = cur_j * p.block_kv + cur_t;
    const bool partial = cur_partial;
    const char* kt = smem + stage * 2 * T::TILE;
    const char* vt = kt + T::TILE;

    const int32_t* sseg = reinterpret_cast<const int32_t*>(smem + T::SEG_OFF) + stage * KC;
    const uint32_t* dmw = reinterpret_cast<const uint32_t*>(smem + T::DM_OFF) + stage * T::DM_WORDS +
                          (wave * 32 + l32) * T::WPT;  // this row's dense-mask words of the tile
    // The tile is processed in parts of 32 keys (kb), each: Sᵀ, softmax, Oᵀ += Vᵀ Pᵀ.
#pragma unroll
    for (int kb = 0; kb < KC / 32; ++kb) {
      // Element mask, only on blocks of class 1: the band and the sequence end
      // leave row q one run of keys [a, e] of the tile (offsets from k0).
      constexpr float kMasked = PW ? 0.0f : kNegInf;
      auto band_run = [&](int& a, int& e) {
        a = qrow + band.lo - k0;
        e = qrow + band.hi - k0;
        a = a > 0 ? a : 0;
        e = e < p.kv_len - 1 - k0 ? e : p.kv_len - 1 - k0;
        e = e < KC - 1 ? e : KC - 1;
        if (e < a) a = e = KC;  // no key of the tile
      };
      // A part of 32 keys that no row of the wavefront may see (past the
      // band, or all of one document none of its rows belongs to) adds
      // nothing to O or L, so its products and probabilities are skipped
      // (exactly: a masked score's probability is 0).
      if (!dense && partial) {
        int a, e;
        band_run(a, e);
        bool none = a == KC || a > 32 * kb + 31 || e < 32 * kb;
        if constexpr (has_seg) {
          // (the lane-crossing reads are made by every lane, outside any
          // condition: each lane carries one key's id)
          const int kid = sseg[32 * kb + l32];
          const int id0 = __builtin_amdgcn_readfirstlane(kid);
          const bool one_id = __builtin_amdgcn_ballot_w64(kid != id0) == 0;
          none = none || (one_id && id0 != myseg);
        }
        if (__builtin_amdgcn_ballot_w64(!none) == 0) continue;
      }

      // ---- Sᵀ = K Qᵀ: 32 keys x 32 queries ----
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + kb * 32 * T::ROWB + koff[s]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc, 0, 0, 0);
      }

      // sacc[r] is the score of key k0 + 32 kb + 8 (r / 4) + 4 hh + r % 4
      // against query qrow.
      // The general form: every score tested against the run (one unsigned
      // compare), the dense-mask bit and the key's segment id; straight-line code.
      auto apply_mask = [&](auto seg_tag, auto dense_tag) {
        constexpr bool kSeg = decltype(seg_tag)::value;
        constexpr bool kDense = decltype(dense_tag)::value;
        int4 kseg4[4];
        if constexpr (kSeg) {
#pragma unroll
          for (int u = 0; u < 4; ++u) kseg4[u] = *reinterpret_cast<const int4*>(sseg + 32 * kb + 8 * u + 4 * hh);
        }
        // dense mask: bit 8 (r / 4) + r % 4 of this word for score r
        const uint32_t dbits = kDense ? dmw[kb] >> (4 * hh) : 0u;
        int a, e;
        band_run(a, e);
        const uint32_t width = (uint32_t)(e - a);
        const int base = 4 * hh - a;  // offset of element r minus a, up to a constant of r
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = 32 * kb + 8 * (r >> 2) + (r & 3);
          bool ok = (uint32_t)(base + kc) <= width;
          if constexpr (kDense) ok &= (bool)((dbits >> (8 * (r >> 2) + (r & 3))) & 1u);
          if constexpr (kSeg) ok &= kseg4[r >> 2][r & 3] == myseg;
          sacc[r] = ok ? sacc[r] : kMasked;
        }
      };
      // The run alone, for a row that keeps (row_ok) or drops every key of
      // these 32. When each row's run covers all 32 keys or none of them
      // (the usual case away from the diagonal: a block is partial because of
      // a document edge or a sequence end elsewhere in it), a row is kept or
      // dropped whole with one lane mask; only otherwise is every score
      // compared.
      auto apply_run = [&](bool row_ok) {
        int a, e;
        band_run(a, e);
        if (!row_ok) a = e = KC;
        const bool whole = a <= 32 * kb && e >= 32 * kb + 31;
        const bool none = a == KC || a > 32 * kb + 31 || e < 32 * kb;
        if (__builtin_amdgcn_ballot_w64(!(whole || none)) == 0) {
          if (__builtin_amdgcn_ballot_w64(none) != 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = none ? kMasked : sacc[r];
          }
        } else {
          const uint32_t width = (uint32_t)(e - a);
          const int base = 4 * hh - a;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kc = 32 * kb + 8 * (r >> 2) + (r & 3);
            sacc[r] = (uint32_t)(base + kc) <= width ? sacc[r] : kMasked;
          }
        }
      };
      // one variant per kind of mask (dense-mask metadata is never combined
      // with segment ids)
      if (partial) {
        if constexpr (dense) {
          apply_mask(std::false_type{}, std::true_type{});
        } else if constexpr (has_seg) {
          // segment ids of these 32 keys, one per lane (both half-waves read
          // the same 32): when they are all equal, a row keeps them all or
          // none, by its own id
          const int kid = sseg[32 * kb + l32];
          const int id0 = __builtin_amdgcn_readfirstlane(kid);
          if (__builtin_amdgcn_ballot_w64(kid != id0) == 0)
            apply_run(id0 == myseg);
          else
            apply_mask(std::true_type{}, std::false_type{});
        } else {
          apply_run(true);
        }
      }

      bf16x8 pb[2];  // [g]: B operand of Oᵀ += Vᵀ Pᵀ for keys 32 kb + 16 g + ...
      if constexpr (!PW) {
        // Probabilities on the row's current reference, with no max: the sum
        // of the lane's 16 rounded probabilities (needed for L anyway, two per
        // dot instruction) shows whether some score rose more than 40 log2
        // units above the reference. Only then, or while a row has no
        // reference yet, does the wavefront take the reference-raising path.
        auto probs = [&](float mneg) {
#pragma unroll
          for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (__bf16)fast_exp2(__builtin_fmaf(sacc[r], c, mneg));
          float rs = 0.0f;
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const bf16x2x4 pr = __builtin_bit_cast(bf16x2x4, pb[g]);
#pragma unroll
            for (int u = 0; u < 4; ++u) rs = __builtin_amdgcn_fdot2_f32_bf16(pr.v[u], kOnes2, rs, false);
          }
          return rs;
        };
        // (a row with no reference yet gets the offset +inf: its sum is inf
        // or NaN, so it fails the test as well)
        float rs = probs(-mref);
        const bool fast = rs <= kFastLimit;  // false for NaN / inf too
        if (__builtin_amdgcn_ballot_w64(!fast) != 0) {
          float mx = kNegInf;
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
          mx = max_xor32(mx) * c;  // max of these 32 keys, log2 domain (-inf if none allowed)
          const bool raise = mx > mref + kRescaleSlack;
          if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float alpha = raise ? fast_exp2(mref - mx) : 1.0f;
            mref = raise ? mx : mref;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          }
          // rows with nothing allowed yet keep mref = -inf; all their entries are -inf here
          rs = probs(mref == kNegInf ? 0.0f : -mref);
        }
        lsum += rs;
      } else {
        const float cneg = -c * kLog2e;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // silu(c s) / q_len = (c / q_len) * s * sigmoid(c s): the constant
          // factor is applied once to O at the end
          const float sv = sacc[r];
          const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(sv * cneg));
          pb[r >> 3][r & 7] = (__bf16)(sv * sg);
        }
      }

      __builtin_amdgcn_s_setprio(0);

      // ---- Oᵀ += Vᵀ Pᵀ over these 32 keys ----
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int rowbase = (32 * kb + 16 * g) * T::ROWB;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vt + rowbase + voff[0][db]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vt + rowbase + voff[1][db]));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[g], oacc[db], 0, 0, 0);
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

  // ---- O = O / L (softmax) or O c / q_len (pointwise), strided store ----
  float inv = c * p.inv_q_len;  // pointwise: the factor left out of P
  if constexpr (!PW) {
    const float l = sum_xor32(lsum);
    inv = l > 0.0f ? 1.0f / l : 0.0f;
    // log-sum-exp of the row's scores x = scale q·k: the probabilities are
    // 2^(x log2(e) - m) summing to L, so log sum e^x = (m + log2 L) ln 2
    // (-inf for a row with no allowed key)
    if (p.lse != nullptr && hh == 0 && qrow < p.q_len)
      p.lse[b * p.lse_sb + h * p.lse_sh + qrow] = l > 0.0f ? (mref + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : kNegInf;
  }
  if (qrow < p.q_len) {
    OutT* orow = og + (int64_t)qrow * p.o_ss;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * hh;
        store4<OutT>(orow + col, oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                     oacc[db][4 * g + 3] * inv);
      }
  }
}

template <int D, int NW, bool PW, typename OutT, int MK>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.nq * p.B * p.H;
  if (total == 0) return hipSuccess;
  const int64_t per_xcd = (total + 7) / 8;
  // units per group on an XCD (0: no round-robin of units, when their count
  // is not a multiple of 8; then total != 8 * per_xcd): the largest power of
  // two up to 8 whose K/V heads, over all 8 XCDs at once, stay within about
  // half of the 256 MB last-level cache (16 MiB per XCD). Measured at
  // B x H x S x D = 2 x 32 x 8192 x 128 (4 MiB of K/V per head): groups of 4
  // beat 1 by 4% and 8 by 2%; at 1 MiB per head groups of 8 beat 1 by 15-20%;
  // at 16 MiB per head groups of 2 were 37% slower than 1.
  int grouped = 0;
  const int units = p.B * p.kv_heads;
  if (units % 8 == 0) {
    const double kv_unit = 4.0 * p.kv_len * p.head_dim;  // bf16 K and V rows of one K/V head
    grouped = 1;
    while (grouped < 8 && 2 * grouped <= units / 8 && 2 * grouped * kv_unit <= 16.0 * 1024 * 1024) grouped *= 2;
  }
  hipLaunchKernelGGL((splash_fwd_bf16_kernel<D, NW, PW, OutT, MK>), dim3((unsigned)(per_xcd * 8)), dim3(NW * 64), 0,
                     stream, p, (int)total, (int)per_xcd, grouped);
  return hipGetLastError();
}

// Each wavefront owns 32 query rows: block_q / 32 wavefronts per workgroup.
template <int D, bool PW, typename OutT, int MK>
hipError_t launch_bq(const FwdParams& p, hipStream_t stream) {
  if (p.block_q == 64) return launch_one<D, 2, PW, OutT, MK>(p, stream);
  if (p.block_q == 256) return launch_one<D, 8, PW, OutT, MK>(p, stream);
  return launch_one<D, 4, PW, OutT, MK>(p, stream);
}

template <int D, bool PW, typename OutT>
hipError_t launch_mk(const FwdParams& p, hipStream_t stream) {
  if (p.mask_blocks != nullptr) return launch_bq<D, PW, OutT, kDense>(p, stream);
  if (p.q_seg != nullptr) return launch_bq<D, PW, OutT, kSegments>(p, stream);
  return launch_bq<D, PW, OutT, kBandOnly>(p, stream);
}

template <bool PW, typename OutT>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  if (p.head_dim == 64) return launch_mk<64, PW, OutT>(p, stream);
  return launch_mk<128, PW, OutT>(p, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, bool pointwise, bool out_f32, hipStream_t stream) {
  if (fwd_rows64_applies(p, pointwise)) return launch_fwd_rows64(p, out_f32, stream);
  if (pointwise) {
    return out_f32 ? launch_d<true, float>(p, stream) : launch_d<true, __bf16>(p, stream);
  }
  return out_f32 ? launch_d<false, float>(p, stream) : launch_d<false, __bf16>(p, stream);
}

}  // namespace splash
