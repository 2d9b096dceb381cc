// Internal interface between the C-ABI host layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splash.h"

namespace splash {

// A head mask reduced to a band on d = k - q: allowed iff lo <= d <= hi.
// causal sets hi <= 0; an unbounded side uses +-kUnbounded.
constexpr int32_t kUnbounded = 0x3fffffff;
constexpr int kMaxLen = 1 << 30;

struct HeadBand {
  int32_t lo;
  int32_t hi;
};

// Host side, shared by the C-ABI translation units (defined in api.cpp).
// Records a failure for splash_last_error() and returns s.
splash_status record_error(splash_status s, const char* fmt, ...);
// Clears the last error and returns SPLASH_OK.
splash_status record_ok();
// Band of one head mask; false (and a recorded error) for invalid fields.
bool head_band(const splash_head_mask& m, int index, HeadBand* out);

struct MaskInfoParams {
  int B, H, q_len, kv_len, block_q, block_kv;
  int nq, nk, meta_batch, meta_heads;
  const int32_t* q_seg;   // [B, q_len] or null
  const int32_t* kv_seg;  // [B, kv_len] or null
  int8_t* block_mask;
  int32_t* data_next;
  // 0: [meta_batch, meta_heads, nq, nk] (rows of kv blocks, the forward's
  // walk); 1: [meta_batch, meta_heads, nk, nq] (columns of q blocks, the
  // dK/dV walk), data_next then running along q blocks
  int columns;
  HeadBand band[SPLASH_MAX_MASK_HEADS];
};

struct FwdParams {
  int B, H, q_len, kv_len, head_dim;
  int band_heads;    // head masks in band[] (1: shared by every head)
  int kv_heads;      // K/V heads; query head h reads kv head h / kv_group
  int kv_group;      // H / kv_heads
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  float scale_log2;  // softmax: scale * log2(e); pointwise: scale * log2(e)
  float scale;       // raw score scale
  float inv_q_len;   // pointwise divisor 1 / q_len
  int block_q, block_kv, nq, nk;
  int meta_heads;    // 1 or H
  int meta_batch;    // 1 or B
  const int8_t* block_mask;
  const int32_t* data_next;
  const int32_t* q_seg;
  const int32_t* kv_seg;
  // dense masks: for a partial block, mask_next names its entry of
  // mask_blocks ([num_mask_blocks][block_q][block_kv / 32] bits); null if none
  const int32_t* mask_next;
  const uint32_t* mask_blocks;
  int64_t num_mask_blocks;
  // softmax: per-row log-sum-exp [B, H, q_len] (rows contiguous), or null
  float* lse;
  int64_t lse_sb, lse_sh;
  HeadBand band[SPLASH_MAX_MASK_HEADS];
};

// Pointwise backward: dQ over the row walk (data_next along kv blocks), dK
// and dV over the column walk (data_next along q blocks).
struct BwdParams {
  int B, H, q_len, kv_len, head_dim;
  int band_heads;    // head masks in band[] (1: shared by every head)
  int kv_heads;      // K/V heads; query head h reads kv head h / kv_group
  int kv_group;      // H / kv_heads
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t do_sb, do_sh, do_ss;
  int64_t dq_sb, dq_sh, dq_ss;
  int64_t dk_sb, dk_sh, dk_ss;
  int64_t dv_sb, dv_sh, dv_ss;
  float scale;       // score scale
  float inv_q_len;   // 1 / q_len
  int meta_batch;    // 1 or B, both walks
  // row walk (dQ): [meta_batch, meta_heads, nq, nk]
  int block_q, block_kv, nq, nk, meta_heads;
  const int8_t* block_mask;
  const int32_t* data_next;
  // column walk (dK, dV): [meta_batch, c_meta_heads, c_nk, c_nq] (columns contiguous)
  int c_block_q, c_block_kv, c_nq, c_nk, c_meta_heads;
  const int8_t* c_block_mask;
  const int32_t* c_data_next;
  const int32_t* q_seg;
  const int32_t* kv_seg;
  // dense masks: for a partial block, mask_next (in its walk's metadata
  // layout) names the block's entry of mask_blocks ([n][block_q][block_kv /
  // 32] bits, the walk's block sizes); null without a dense mask
  const int32_t* mask_next;
  const uint32_t* mask_blocks;
  int64_t num_mask_blocks;
  const int32_t* c_mask_next;
  const uint32_t* c_mask_blocks;
  int64_t c_num_mask_blocks;
  // softmax backward: per-row log-sum-exp of the forward and
  // delta = rowsum(dO * O), both [B, H, q_len] fp32 (rows contiguous)
  int softmax;
  const float* lse;
  const float* delta;
  int64_t st_sb, st_sh;
  HeadBand band[SPLASH_MAX_MASK_HEADS];
};

// delta = rowsum(O * dO) per (b, h, query), fp32.
struct DeltaParams {
  int B, H, q_len, head_dim;
  const void* o;
  const void* d_o;
  float* delta;
  int64_t o_sb, o_sh, o_ss;
  int64_t do_sb, do_sh, do_ss;
  int64_t d_sb, d_sh;
};

// Launchers; return the launch error (hipSuccess when enqueued).
hipError_t launch_mask_info(const MaskInfoParams& p, hipStream_t stream);
// Same classes in the column layout (p.columns = 1), data_next along the q
// blocks of each kv-block column.
hipError_t launch_mask_info_dkv(const MaskInfoParams& p, hipStream_t stream);
// bf16 inputs, matrix-core path. out_f32 selects an fp32 output.
hipError_t launch_fwd_bf16(const FwdParams& p, bool pointwise, bool out_f32, hipStream_t stream);
// The softmax forward at head_dim 128 with 64 query rows per wavefront
// (block_q 128 or 256, no dense-mask store): whether it applies, and its launch.
bool fwd_rows64_applies(const FwdParams& p, bool pointwise);
hipError_t launch_fwd_rows64(const FwdParams& p, bool out_f32, hipStream_t stream);
// fp32 inputs and output.
hipError_t launch_fwd_f32(const FwdParams& p, bool pointwise, hipStream_t stream);
// Pointwise backward, bf16 inputs (gradients bf16 or fp32) and fp32 inputs.
hipError_t launch_pointwise_bwd_bf16(const BwdParams& p, bool out_f32, hipStream_t stream);
hipError_t launch_pointwise_bwd_f32(const BwdParams& p, hipStream_t stream);
// (the softmax backward runs through the same two launchers with p.softmax set)
hipError_t launch_softmax_delta(const DeltaParams& p, bool bf16, hipStream_t stream);

}  // namespace splash
