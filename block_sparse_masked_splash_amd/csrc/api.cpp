// C ABI of libsplash: host-side validation and kernel dispatch.
//
// Every check runs before anything is enqueued; a failed check returns its
// status, records a message for splash_last_error() and touches nothing.
// Error classes follow the argument checks of "hstu_ops.py" (RecML):
// ValueError-style problems (shapes, both-or-neither segment ids) are
// SPLASH_ERR_INVALID_ARGUMENT, NotImplementedError-style ones (a valid request
// without a compiled kernel) are SPLASH_ERR_UNSUPPORTED, and metadata built
// for another call is SPLASH_ERR_METADATA_MISMATCH. There is no fallback path.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "internal.h"

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace splash {

splash_status record_error(splash_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(splash_status_string(s)) + ": " + buf;
  return s;
}

splash_status record_ok() {
  g_last_error.clear();
  return SPLASH_OK;
}

bool head_band(const splash_head_mask& m, int index, HeadBand* out) {
  if (m.causal != 0 && m.causal != 1) {
    record_error(SPLASH_ERR_INVALID_ARGUMENT, "head %d: causal=%d must be 0 or 1", index, m.causal);
    return false;
  }
  if (m.window_left < -1 || m.window_right < -1) {
    record_error(SPLASH_ERR_INVALID_ARGUMENT, "head %d: window bounds must be >= -1", index);
    return false;
  }
  int32_t lo = m.window_left >= 0 ? -m.window_left : -kUnbounded;
  int32_t hi = m.window_right >= 0 ? m.window_right : kUnbounded;
  if (m.causal && hi > 0) hi = 0;
  if (lo < -kUnbounded) lo = -kUnbounded;
  if (hi > kUnbounded) hi = kUnbounded;
  *out = {lo, hi};
  return true;
}

}  // namespace splash

namespace {

using splash::record_error;
splash_status ok() { return splash::record_ok(); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool len_ok(int x) { return x >= 0 && x <= splash::kMaxLen; }

// Metadata, segment ids and row statistics are read as aligned 32-bit words.
bool misaligned4(const void* p) { return p != nullptr && reinterpret_cast<uintptr_t>(p) % 4 != 0; }

// Checks the mask description against B and H; fills the head bands.
splash_status check_mask(int H, const splash_mask_desc* mask, splash::HeadBand* band) {
  if (mask == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "mask is null");
  const int nm = mask->num_mask_heads;
  if (nm < 1 || nm > SPLASH_MAX_MASK_HEADS)
    return record_error(nm < 1 ? SPLASH_ERR_INVALID_ARGUMENT : SPLASH_ERR_UNSUPPORTED,
                "num_mask_heads=%d must be 1 or H, at most %d", nm, SPLASH_MAX_MASK_HEADS);
  if (nm != 1 && nm != H) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "num_mask_heads=%d is neither 1 nor H=%d", nm, H);
  if (mask->heads == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "mask->heads is null");
  if ((mask->q_segment_ids == nullptr) != (mask->kv_segment_ids == nullptr))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "both or neither of q_segment_ids and kv_segment_ids must be given");
  if (misaligned4(mask->q_segment_ids) || misaligned4(mask->kv_segment_ids))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "segment ids must be 4-byte aligned");
  for (int h = 0; h < nm; ++h)
    if (!splash::head_band(mask->heads[h], h, &band[h])) return SPLASH_ERR_INVALID_ARGUMENT;
  return SPLASH_OK;
}

splash_status check_sizes(int B, int H, int q_len, int kv_len) {
  if (B < 0 || H < 0 || !len_ok(q_len) || !len_ok(kv_len) || B > (1 << 24) || H > (1 << 16))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "bad sizes B=%d H=%d q_len=%d kv_len=%d", B, H, q_len, kv_len);
  return SPLASH_OK;
}

splash_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return record_error(SPLASH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

splash_status check_tensor(const char* name, const void* ptr, const int64_t* strides, int elem_bytes,
                           bool needed) {
  if (strides == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s strides are null", name);
  if (!needed) return SPLASH_OK;
  if (ptr == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s is null", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  for (int a = 0; a < 3; ++a) {
    if (strides[a] < 0) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s stride %d is negative", name, a);
    if ((strides[a] * elem_bytes) % 16 != 0)
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s stride %d (%lld elements) breaks 16-byte row alignment", name, a,
                  (long long)strides[a]);
  }
  // tiles of up to 64 rows are copied through buffer resources whose offsets
  // and sizes are 32-bit: rows must lie less than 64 MiB apart
  if (strides[2] * elem_bytes >= ((int64_t)1 << 26))
    return record_error(SPLASH_ERR_UNSUPPORTED, "%s rows are %lld bytes apart (at most 64 MiB - 16 supported)", name,
                        (long long)(strides[2] * elem_bytes));
  return SPLASH_OK;
}

splash_status fwd_common(bool pointwise, splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                         int q_len, int kv_len, int head_dim, const void* q, const int64_t q_strides[3], const void* k,
                         const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* o,
                         const int64_t o_strides[3], float scale, const splash_mask_desc* mask,
                         const splash_mask_info* info, const splash_partial_masks* partial, float* lse,
                         const int64_t* lse_strides, hipStream_t stream) {
  splash_status s = check_sizes(B, H, q_len, kv_len);
  if (s != SPLASH_OK) return s;
  if (kv_heads < 1 || kv_heads > H || H % kv_heads != 0)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "kv_heads=%d must divide H=%d", kv_heads, H);
  const bool f32 = in_dtype == SPLASH_F32 && out_dtype == SPLASH_F32;
  const bool bf16 = in_dtype == SPLASH_BF16 && (out_dtype == SPLASH_BF16 || out_dtype == SPLASH_F32);
  if (!f32 && !bf16)
    return record_error(SPLASH_ERR_UNSUPPORTED, "dtype pair in=%d out=%d (supported: f32->f32, bf16->bf16, bf16->f32)",
                (int)in_dtype, (int)out_dtype);
  if (head_dim <= 0) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "head_dim=%d", head_dim);
  if (head_dim != 64 && head_dim != 128)
    return record_error(SPLASH_ERR_UNSUPPORTED, "head_dim=%d (supported: 64, 128)", head_dim);
  if (!std::isfinite(scale)) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "scale is not finite");

  splash::FwdParams p{};
  s = check_mask(H, mask, p.band);
  if (s != SPLASH_OK) return s;
  if (info == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "info is null");

  const bool work = (int64_t)B * H * q_len > 0;
  const int in_bytes = in_dtype == SPLASH_F32 ? 4 : 2;
  const int out_bytes = out_dtype == SPLASH_F32 ? 4 : 2;
  if ((s = check_tensor("q", q, q_strides, in_bytes, work)) != SPLASH_OK) return s;
  if ((s = check_tensor("k", k, k_strides, in_bytes, work && kv_len > 0)) != SPLASH_OK) return s;
  if ((s = check_tensor("v", v, v_strides, in_bytes, work && kv_len > 0)) != SPLASH_OK) return s;
  if ((s = check_tensor("o", o, o_strides, out_bytes, work)) != SPLASH_OK) return s;
  if (lse_strides != nullptr) {  // log-sum-exp requested (softmax only)
    if (pointwise) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "log-sum-exp is defined for softmax only");
    if (work && lse == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse is null");
    if (misaligned4(lse)) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    if (lse_strides[0] < 0 || lse_strides[1] < 0)
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse strides must be >= 0");
  }

  const bool seg = mask->q_segment_ids != nullptr;
  const int bq = info->block_q, bkv = info->block_kv;
  if (bq <= 0 || bkv <= 0) return record_error(SPLASH_ERR_METADATA_MISMATCH, "info block sizes %d x %d", bq, bkv);
  const int64_t nq = ceil_div(q_len, bq), nk = ceil_div(kv_len, bkv);
  // metadata heads: those of the head masks, or (dense masks) 1 or H with the
  // head masks 1 or as many
  const int nm = mask->num_mask_heads;
  const bool heads_ok = partial == nullptr ? info->meta_heads == nm
                                           : ((info->meta_heads == 1 || info->meta_heads == H) &&
                                              (nm == 1 || nm == info->meta_heads));
  if (info->meta_batch != (seg ? B : 1) || !heads_ok || info->num_q_blocks != nq || info->num_kv_blocks != nk)
    return record_error(SPLASH_ERR_METADATA_MISMATCH,
                "info [%d,%d,%d,%d] but this call needs [%d,%d,%lld,%lld] (segment ids %s%s)", info->meta_batch,
                info->meta_heads, info->num_q_blocks, info->num_kv_blocks, seg ? B : 1, nm, (long long)nq,
                (long long)nk, seg ? "given" : "absent", partial ? ", dense masks" : "");
  if ((bq != 64 && bq != 128 && bq != 256) || (bkv != 64 && bkv != 128))
    return record_error(SPLASH_ERR_UNSUPPORTED, "block sizes %d x %d (supported: block_q 64, 128 or 256; block_kv 64 or 128)",
                bq, bkv);
  if (work && nk > 0 && (info->block_mask == nullptr || info->data_next == nullptr))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "info arrays are null");
  if (misaligned4(info->block_mask) || misaligned4(info->data_next))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "info arrays must be 4-byte aligned");
  if (partial != nullptr) {
    if (partial->num_blocks < 0 || partial->num_blocks > ((int64_t)1 << 31))
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "num_blocks=%lld", (long long)partial->num_blocks);
    if (work && nk > 0 && (partial->mask_next == nullptr || (partial->num_blocks > 0 && partial->mask_blocks == nullptr)))
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "dense mask arrays are null");
    if (misaligned4(partial->mask_next) || misaligned4(partial->mask_blocks))
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "dense mask arrays must be 4-byte aligned");
  }
  if (!work) return ok();
  if (nq * B * H >= (int64_t)1 << 31)
    return record_error(SPLASH_ERR_UNSUPPORTED, "%lld workgroups exceed one launch", (long long)(nq * B * H));

  p.B = B;
  p.H = H;
  p.band_heads = nm;
  p.kv_heads = kv_heads;
  p.kv_group = H / kv_heads;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.head_dim = head_dim;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.q_sb = q_strides[0], p.q_sh = q_strides[1], p.q_ss = q_strides[2];
  p.k_sb = k_strides[0], p.k_sh = k_strides[1], p.k_ss = k_strides[2];
  p.v_sb = v_strides[0], p.v_sh = v_strides[1], p.v_ss = v_strides[2];
  p.o_sb = o_strides[0], p.o_sh = o_strides[1], p.o_ss = o_strides[2];
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.inv_q_len = 1.0f / (float)q_len;
  p.block_q = bq;
  p.block_kv = bkv;
  p.nq = (int)nq;
  p.nk = (int)nk;
  p.meta_heads = info->meta_heads;
  p.meta_batch = seg ? B : 1;
  p.block_mask = info->block_mask;
  p.data_next = info->data_next;
  // with a dense mask, segment ids are folded into the host-built classes and
  // partial-block bits (metadata per batch row), so the kernel does not read them
  p.q_seg = partial != nullptr ? nullptr : mask->q_segment_ids;
  p.kv_seg = partial != nullptr ? nullptr : mask->kv_segment_ids;
  if (lse_strides != nullptr) {
    p.lse = lse;
    p.lse_sb = lse_strides[0];
    p.lse_sh = lse_strides[1];
  }
  if (partial != nullptr) {
    p.mask_next = partial->mask_next;
    p.mask_blocks = partial->num_blocks > 0 ? partial->mask_blocks : nullptr;
    p.num_mask_blocks = partial->num_blocks;
  }

  hipError_t e = f32 ? splash::launch_fwd_f32(p, pointwise, stream)
                     : splash::launch_fwd_bf16(p, pointwise, out_dtype == SPLASH_F32, stream);
  return hip_status(e, pointwise ? "pointwise forward launch" : "softmax forward launch");
}

// Checks one metadata struct against the call; `what` names it in messages.
splash_status check_info(const char* what, const splash_mask_info* info, int B, int H, int q_len, int kv_len,
                         bool seg, int nm, bool work, bool dense = false) {
  if (info == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s is null", what);
  const int bq = info->block_q, bkv = info->block_kv;
  if (bq <= 0 || bkv <= 0)
    return record_error(SPLASH_ERR_METADATA_MISMATCH, "%s block sizes %d x %d", what, bq, bkv);
  const int64_t nq = ceil_div(q_len, bq), nk = ceil_div(kv_len, bkv);
  // metadata heads: those of the head masks, or (dense masks) 1 or H with the
  // head masks 1 or as many
  const bool heads_ok = !dense ? info->meta_heads == nm
                               : ((info->meta_heads == 1 || info->meta_heads == H) && (nm == 1 || nm == info->meta_heads));
  if (info->meta_batch != (seg ? B : 1) || !heads_ok || info->num_q_blocks != nq || info->num_kv_blocks != nk)
    return record_error(SPLASH_ERR_METADATA_MISMATCH,
                        "%s [%d,%d,%d,%d] but this call needs [%d,%d,%lld,%lld] (segment ids %s)", what,
                        info->meta_batch, info->meta_heads, info->num_q_blocks, info->num_kv_blocks, seg ? B : 1, nm,
                        (long long)nq, (long long)nk, seg ? "given" : "absent");
  if (work && nq > 0 && nk > 0 && (info->block_mask == nullptr || info->data_next == nullptr))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s arrays are null", what);
  if (misaligned4(info->block_mask) || misaligned4(info->data_next))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s arrays must be 4-byte aligned", what);
  return SPLASH_OK;
}

// Checks the dense-mask arrays of one walk (`what` names them in messages).
splash_status check_partial(const char* what, const splash_partial_masks* partial, bool work) {
  if (partial->num_blocks < 0 || partial->num_blocks > ((int64_t)1 << 31))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s num_blocks=%lld", what, (long long)partial->num_blocks);
  if (work && (partial->mask_next == nullptr || (partial->num_blocks > 0 && partial->mask_blocks == nullptr)))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s dense mask arrays are null", what);
  if (misaligned4(partial->mask_next) || misaligned4(partial->mask_blocks))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "%s dense mask arrays must be 4-byte aligned", what);
  return SPLASH_OK;
}

splash_status bwd_common(bool softmax, splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                         int q_len, int kv_len, int head_dim, const void* q, const int64_t q_strides[3], const void* k,
                         const int64_t k_strides[3], const void* v, const int64_t v_strides[3], const void* d_o,
                         const int64_t do_strides[3], const float* lse, const float* delta,
                         const int64_t* stat_strides, void* dq, const int64_t dq_strides[3], void* dk,
                         const int64_t dk_strides[3], void* dv, const int64_t dv_strides[3], float scale,
                         const splash_mask_desc* mask, const splash_mask_info* info,
                         const splash_mask_info* info_dkv, hipStream_t stream,
                         const splash_partial_masks* partial = nullptr,
                         const splash_partial_masks* partial_dkv = nullptr) {
  splash_status s = check_sizes(B, H, q_len, kv_len);
  if (s != SPLASH_OK) return s;
  if (kv_heads < 1 || kv_heads > H || H % kv_heads != 0)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "kv_heads=%d must divide H=%d", kv_heads, H);
  const bool f32 = in_dtype == SPLASH_F32 && out_dtype == SPLASH_F32;
  const bool bf16 = in_dtype == SPLASH_BF16 && (out_dtype == SPLASH_BF16 || out_dtype == SPLASH_F32);
  if (!f32 && !bf16)
    return record_error(SPLASH_ERR_UNSUPPORTED, "dtype pair in=%d out=%d (supported: f32->f32, bf16->bf16, bf16->f32)",
                        (int)in_dtype, (int)out_dtype);
  if (head_dim <= 0) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "head_dim=%d", head_dim);
  if (head_dim != 64 && head_dim != 128)
    return record_error(SPLASH_ERR_UNSUPPORTED, "head_dim=%d (supported: 64, 128)", head_dim);
  if (!std::isfinite(scale)) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "scale is not finite");

  splash::BwdParams p{};
  s = check_mask(H, mask, p.band);
  if (s != SPLASH_OK) return s;
  const bool seg = mask->q_segment_ids != nullptr;
  const int nm = mask->num_mask_heads;
  const bool qwork = (int64_t)B * H * q_len > 0;
  const bool kwork = (int64_t)B * kv_heads * kv_len > 0;
  const bool work = qwork || kwork;
  if ((partial == nullptr) != (partial_dkv == nullptr))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "both or neither of partial and partial_dkv must be given");
  const bool dense = partial != nullptr;
  if ((s = check_info("info", info, B, H, q_len, kv_len, seg, nm, work, dense)) != SPLASH_OK) return s;
  if ((s = check_info("info_dkv", info_dkv, B, H, q_len, kv_len, seg, nm, work, dense)) != SPLASH_OK) return s;
  if (dense) {
    if (info->meta_heads != info_dkv->meta_heads)
      return record_error(SPLASH_ERR_METADATA_MISMATCH, "info and info_dkv have %d and %d metadata heads",
                          info->meta_heads, info_dkv->meta_heads);
    if ((s = check_partial("partial", partial, work)) != SPLASH_OK) return s;
    if ((s = check_partial("partial_dkv", partial_dkv, work)) != SPLASH_OK) return s;
    if (info->block_kv % 32 != 0 || info_dkv->block_kv % 32 != 0)
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "dense-mask metadata needs block_kv a multiple of 32");
  }
  const int bq = info->block_q, bkv = info->block_kv;
  if ((bq != 64 && bq != 128 && bq != 256) || (bkv != 64 && bkv != 128))
    return record_error(SPLASH_ERR_UNSUPPORTED, "info block sizes %d x %d (supported: block_q 64, 128 or 256; "
                        "block_kv 64 or 128)", bq, bkv);
  const int cbq = info_dkv->block_q, cbkv = info_dkv->block_kv;
  if (cbq % 32 != 0 || cbq > 1024 || (cbkv != 64 && cbkv != 128))
    return record_error(SPLASH_ERR_UNSUPPORTED, "info_dkv block sizes %d x %d (supported: block_q a multiple of 32 "
                        "up to 1024; block_kv 64 or 128)", cbq, cbkv);

  const int in_bytes = in_dtype == SPLASH_F32 ? 4 : 2;
  const int out_bytes = out_dtype == SPLASH_F32 ? 4 : 2;
  const bool both = qwork && kwork;  // q-side and kv-side rows exist
  if ((s = check_tensor("q", q, q_strides, in_bytes, both)) != SPLASH_OK) return s;
  if ((s = check_tensor("k", k, k_strides, in_bytes, both)) != SPLASH_OK) return s;
  if ((s = check_tensor("v", v, v_strides, in_bytes, both)) != SPLASH_OK) return s;
  if ((s = check_tensor("d_o", d_o, do_strides, in_bytes, both)) != SPLASH_OK) return s;
  if ((s = check_tensor("dq", dq, dq_strides, out_bytes, qwork)) != SPLASH_OK) return s;
  if ((s = check_tensor("dk", dk, dk_strides, out_bytes, kwork)) != SPLASH_OK) return s;
  if ((s = check_tensor("dv", dv, dv_strides, out_bytes, kwork)) != SPLASH_OK) return s;
  if (softmax) {
    if (stat_strides == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse / delta strides are null");
    if (stat_strides[0] < 0 || stat_strides[1] < 0)
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse / delta strides must be >= 0");
    if (both && (lse == nullptr || delta == nullptr))
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse or delta is null");
    if (both && (reinterpret_cast<uintptr_t>(lse) % 4 != 0 || reinterpret_cast<uintptr_t>(delta) % 4 != 0))
      return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse and delta must be 4-byte aligned");
  }
  if (!work) return ok();
  const int64_t nq = ceil_div(q_len, bq), nk = ceil_div(kv_len, bkv);
  const int64_t cnq = ceil_div(q_len, cbq), cnk = ceil_div(kv_len, cbkv);
  // (the dK/dV pass may split a kv block over up to block_kv / 32 workgroups)
  if (nq * B * H >= (int64_t)1 << 31 || cnk * (cbkv / 32 > 1 ? cbkv / 32 : 1) * B * kv_heads >= (int64_t)1 << 31)
    return record_error(SPLASH_ERR_UNSUPPORTED, "too many workgroups for one launch");

  p.B = B;
  p.H = H;
  p.band_heads = nm;
  p.kv_heads = kv_heads;
  p.kv_group = H / kv_heads;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.head_dim = head_dim;
  p.q = q;
  p.k = k;
  p.v = v;
  p.d_o = d_o;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.q_sb = q_strides[0], p.q_sh = q_strides[1], p.q_ss = q_strides[2];
  p.k_sb = k_strides[0], p.k_sh = k_strides[1], p.k_ss = k_strides[2];
  p.v_sb = v_strides[0], p.v_sh = v_strides[1], p.v_ss = v_strides[2];
  p.do_sb = do_strides[0], p.do_sh = do_strides[1], p.do_ss = do_strides[2];
  p.dq_sb = dq_strides[0], p.dq_sh = dq_strides[1], p.dq_ss = dq_strides[2];
  p.dk_sb = dk_strides[0], p.dk_sh = dk_strides[1], p.dk_ss = dk_strides[2];
  p.dv_sb = dv_strides[0], p.dv_sh = dv_strides[1], p.dv_ss = dv_strides[2];
  p.scale = scale;
  p.inv_q_len = q_len > 0 ? 1.0f / (float)q_len : 0.0f;
  p.meta_batch = seg ? B : 1;
  p.block_q = bq;
  p.block_kv = bkv;
  p.nq = (int)nq;
  p.nk = (int)nk;
  p.meta_heads = info->meta_heads;
  p.block_mask = info->block_mask;
  p.data_next = info->data_next;
  p.c_block_q = cbq;
  p.c_block_kv = cbkv;
  p.c_nq = (int)cnq;
  p.c_nk = (int)cnk;
  p.c_meta_heads = info_dkv->meta_heads;
  p.c_block_mask = info_dkv->block_mask;
  p.c_data_next = info_dkv->data_next;
  // with a dense mask, segment ids are folded into the host-built metadata
  p.q_seg = dense ? nullptr : mask->q_segment_ids;
  p.kv_seg = dense ? nullptr : mask->kv_segment_ids;
  if (dense) {
    p.mask_next = partial->mask_next;
    p.mask_blocks = partial->num_blocks > 0 ? partial->mask_blocks : nullptr;
    p.num_mask_blocks = partial->num_blocks;
    p.c_mask_next = partial_dkv->mask_next;
    p.c_mask_blocks = partial_dkv->num_blocks > 0 ? partial_dkv->mask_blocks : nullptr;
    p.c_num_mask_blocks = partial_dkv->num_blocks;
  }
  p.softmax = softmax ? 1 : 0;
  if (softmax) {
    p.lse = lse;
    p.delta = delta;
    p.st_sb = stat_strides[0];
    p.st_sh = stat_strides[1];
  }
  hipError_t e = f32 ? splash::launch_pointwise_bwd_f32(p, stream)
                     : splash::launch_pointwise_bwd_bf16(p, out_dtype == SPLASH_F32, stream);
  return hip_status(e, softmax ? "softmax backward launch" : "pointwise backward launch");
}

splash_status mask_info_common(bool dkv, int B, int H, int q_len, int kv_len, int block_q, int block_kv,
                               const splash_mask_desc* mask, const splash_mask_info* info, hipStream_t stream);

}  // namespace

extern "C" {

const char* splash_status_string(splash_status s) {
  switch (s) {
    case SPLASH_OK: return "SPLASH_OK";
    case SPLASH_ERR_INVALID_ARGUMENT: return "SPLASH_ERR_INVALID_ARGUMENT";
    case SPLASH_ERR_UNSUPPORTED: return "SPLASH_ERR_UNSUPPORTED";
    case SPLASH_ERR_METADATA_MISMATCH: return "SPLASH_ERR_METADATA_MISMATCH";
    case SPLASH_ERR_HIP: return "SPLASH_ERR_HIP";
  }
  return "SPLASH_ERR_UNKNOWN";
}

const char* splash_last_error(void) { return g_last_error.c_str(); }

int splash_abi_version(void) { return SPLASH_ABI_VERSION; }

size_t splash_mask_info_entries(int B, int H, int q_len, int kv_len, int block_q, int block_kv,
                                const splash_mask_desc* mask) {
  if (B < 0 || H < 0 || !len_ok(q_len) || !len_ok(kv_len)) return 0;
  if (block_q < 1 || block_q > 1024 || block_kv < 1 || block_kv > 1024) return 0;
  if (mask == nullptr || (mask->num_mask_heads != 1 && mask->num_mask_heads != H)) return 0;
  if (mask->num_mask_heads < 1 || mask->num_mask_heads > SPLASH_MAX_MASK_HEADS) return 0;
  if ((mask->q_segment_ids == nullptr) != (mask->kv_segment_ids == nullptr)) return 0;
  const int64_t bm = mask->q_segment_ids ? B : 1;
  return (size_t)(bm * mask->num_mask_heads * ceil_div(q_len, block_q) * ceil_div(kv_len, block_kv));
}

splash_status splash_mask_info_build(int B, int H, int q_len, int kv_len, int block_q, int block_kv,
                                     const splash_mask_desc* mask, const splash_mask_info* info,
                                     hipStream_t stream) {
  return mask_info_common(false, B, H, q_len, kv_len, block_q, block_kv, mask, info, stream);
}

splash_status splash_mask_info_build_dkv(int B, int H, int q_len, int kv_len, int block_q, int block_kv,
                                         const splash_mask_desc* mask, const splash_mask_info* info,
                                         hipStream_t stream) {
  return mask_info_common(true, B, H, q_len, kv_len, block_q, block_kv, mask, info, stream);
}

splash_status splash_pointwise_bwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                                   int q_len, int kv_len, int head_dim, const void* q, const int64_t q_strides[3],
                                   const void* k, const int64_t k_strides[3], const void* v,
                                   const int64_t v_strides[3], const void* d_o, const int64_t do_strides[3],
                                   void* dq, const int64_t dq_strides[3], void* dk, const int64_t dk_strides[3],
                                   void* dv, const int64_t dv_strides[3], float scale,
                                   const splash_mask_desc* mask, const splash_mask_info* info,
                                   const splash_mask_info* info_dkv, hipStream_t stream) {
  return bwd_common(false, in_dtype, out_dtype, B, H, kv_heads, q_len, kv_len, head_dim, q, q_strides, k, k_strides,
                    v, v_strides, d_o, do_strides, nullptr, nullptr, nullptr, dq, dq_strides, dk, dk_strides, dv,
                    dv_strides, scale, mask, info, info_dkv, stream);
}

splash_status splash_softmax_bwd_preprocess(splash_dtype dtype, int B, int H, int q_len, int head_dim,
                                            const void* o, const int64_t o_strides[3], const void* d_o,
                                            const int64_t do_strides[3], float* delta,
                                            const int64_t delta_strides[2], hipStream_t stream) {
  if (B < 0 || H < 0 || !len_ok(q_len))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "bad sizes B=%d H=%d q_len=%d", B, H, q_len);
  if (dtype != SPLASH_F32 && dtype != SPLASH_BF16) return record_error(SPLASH_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return record_error(head_dim <= 0 ? SPLASH_ERR_INVALID_ARGUMENT : SPLASH_ERR_UNSUPPORTED,
                        "head_dim=%d (supported: 64, 128)", head_dim);
  const bool work = (int64_t)B * H * q_len > 0;
  const int eb = dtype == SPLASH_F32 ? 4 : 2;
  splash_status s;
  if ((s = check_tensor("o", o, o_strides, eb, work)) != SPLASH_OK) return s;
  if ((s = check_tensor("d_o", d_o, do_strides, eb, work)) != SPLASH_OK) return s;
  if (delta_strides == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "delta strides are null");
  if (delta_strides[0] < 0 || delta_strides[1] < 0)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "delta strides must be >= 0");
  if (work && (delta == nullptr || reinterpret_cast<uintptr_t>(delta) % 4 != 0))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "delta is null or not 4-byte aligned");
  if (!work) return ok();
  splash::DeltaParams p{};
  p.B = B;
  p.H = H;
  p.q_len = q_len;
  p.head_dim = head_dim;
  p.o = o;
  p.d_o = d_o;
  p.delta = delta;
  p.o_sb = o_strides[0], p.o_sh = o_strides[1], p.o_ss = o_strides[2];
  p.do_sb = do_strides[0], p.do_sh = do_strides[1], p.do_ss = do_strides[2];
  p.d_sb = delta_strides[0], p.d_sh = delta_strides[1];
  return hip_status(splash::launch_softmax_delta(p, dtype == SPLASH_BF16, stream), "softmax delta launch");
}

splash_status splash_softmax_bwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                                 int q_len, int kv_len, int head_dim, const void* q, const int64_t q_strides[3],
                                 const void* k, const int64_t k_strides[3], const void* v,
                                 const int64_t v_strides[3], const void* d_o, const int64_t do_strides[3],
                                 const float* lse, const float* delta, const int64_t stat_strides[2], void* dq,
                                 const int64_t dq_strides[3], void* dk, const int64_t dk_strides[3], void* dv,
                                 const int64_t dv_strides[3], float scale, const splash_mask_desc* mask,
                                 const splash_mask_info* info, const splash_mask_info* info_dkv,
                                 hipStream_t stream) {
  return bwd_common(true, in_dtype, out_dtype, B, H, kv_heads, q_len, kv_len, head_dim, q, q_strides, k, k_strides, v,
                    v_strides, d_o, do_strides, lse, delta, stat_strides, dq, dq_strides, dk, dk_strides, dv,
                    dv_strides, scale, mask, info, info_dkv, stream);
}

}  // extern "C"

namespace {

splash_status mask_info_common(bool dkv, int B, int H, int q_len, int kv_len, int block_q, int block_kv,
                               const splash_mask_desc* mask, const splash_mask_info* info, hipStream_t stream) {
  splash_status s = check_sizes(B, H, q_len, kv_len);
  if (s != SPLASH_OK) return s;
  if (block_q < 1 || block_q > 1024 || block_kv < 1 || block_kv > 1024)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "block sizes %d x %d must be in [1, 1024]", block_q, block_kv);
  splash::MaskInfoParams p{};
  s = check_mask(H, mask, p.band);
  if (s != SPLASH_OK) return s;
  if (info == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "info is null");
  const bool seg = mask->q_segment_ids != nullptr;
  const int64_t nq = ceil_div(q_len, block_q), nk = ceil_div(kv_len, block_kv);
  if (info->meta_batch != (seg ? B : 1) || info->meta_heads != mask->num_mask_heads || info->num_q_blocks != nq ||
      info->num_kv_blocks != nk || info->block_q != block_q || info->block_kv != block_kv)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "info fields [%d,%d,%d,%d] blocks %dx%d do not describe this call",
                info->meta_batch, info->meta_heads, info->num_q_blocks, info->num_kv_blocks, info->block_q,
                info->block_kv);
  const int64_t entries = (int64_t)info->meta_batch * info->meta_heads * nq * nk;
  if (entries == 0) return ok();
  if ((int64_t)info->meta_batch * info->meta_heads * nq / 4 >= ((int64_t)1 << 31) ||
      (int64_t)info->meta_batch * info->meta_heads * nk / 4 >= ((int64_t)1 << 31))
    return record_error(SPLASH_ERR_UNSUPPORTED, "too many metadata rows for one launch");
  // the segment-id classification runs one wavefront per 64 entries of a row
  // (or column), four wavefronts per workgroup
  if (seg) {
    const int64_t lines = (int64_t)info->meta_batch * info->meta_heads * (dkv ? nk : nq);
    const int64_t waves = lines * ceil_div(dkv ? nq : nk, 64);
    if (waves / 4 >= ((int64_t)1 << 31))
      return record_error(SPLASH_ERR_UNSUPPORTED, "too many metadata entries for one launch");
  }
  if (info->block_mask == nullptr || info->data_next == nullptr)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "info arrays are null");
  if (misaligned4(info->block_mask) || misaligned4(info->data_next))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "info arrays must be 4-byte aligned");
  p.B = B;
  p.H = H;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.block_q = block_q;
  p.block_kv = block_kv;
  p.nq = (int)nq;
  p.nk = (int)nk;
  p.meta_batch = info->meta_batch;
  p.meta_heads = info->meta_heads;
  p.q_seg = mask->q_segment_ids;
  p.kv_seg = mask->kv_segment_ids;
  p.block_mask = info->block_mask;
  p.data_next = info->data_next;
  p.columns = dkv ? 1 : 0;
  return dkv ? hip_status(splash::launch_mask_info_dkv(p, stream), "splash_mask_info_build_dkv launch")
             : hip_status(splash::launch_mask_info(p, stream), "splash_mask_info_build launch");
}

}  // namespace

extern "C" {

splash_status splash_fwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int q_len, int kv_len,
                         int head_dim, const void* q, const int64_t q_strides[3], const void* k,
                         const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* o,
                         const int64_t o_strides[3], float scale, const splash_mask_desc* mask,
                         const splash_mask_info* info, hipStream_t stream) {
  return fwd_common(false, in_dtype, out_dtype, B, H, H, q_len, kv_len, head_dim, q, q_strides, k, k_strides, v,
                    v_strides, o, o_strides, scale, mask, info, nullptr, nullptr, nullptr, stream);
}

splash_status splash_pointwise_fwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int q_len,
                                   int kv_len, int head_dim, const void* q, const int64_t q_strides[3],
                                   const void* k, const int64_t k_strides[3], const void* v,
                                   const int64_t v_strides[3], void* o, const int64_t o_strides[3], float scale,
                                   const splash_mask_desc* mask, const splash_mask_info* info,
                                   hipStream_t stream) {
  return fwd_common(true, in_dtype, out_dtype, B, H, H, q_len, kv_len, head_dim, q, q_strides, k, k_strides, v,
                    v_strides, o, o_strides, scale, mask, info, nullptr, nullptr, nullptr, stream);
}

splash_status splash_gqa_fwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads, int q_len,
                             int kv_len, int head_dim, const void* q, const int64_t q_strides[3], const void* k,
                             const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* o,
                             const int64_t o_strides[3], float scale, const splash_mask_desc* mask,
                             const splash_mask_info* info, hipStream_t stream) {
  return fwd_common(false, in_dtype, out_dtype, B, H, kv_heads, q_len, kv_len, head_dim, q, q_strides, k, k_strides,
                    v, v_strides, o, o_strides, scale, mask, info, nullptr, nullptr, nullptr, stream);
}

splash_status splash_gqa_pointwise_fwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                                       int q_len, int kv_len, int head_dim, const void* q,
                                       const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                                       const void* v, const int64_t v_strides[3], void* o,
                                       const int64_t o_strides[3], float scale, const splash_mask_desc* mask,
                                       const splash_mask_info* info, hipStream_t stream) {
  return fwd_common(true, in_dtype, out_dtype, B, H, kv_heads, q_len, kv_len, head_dim, q, q_strides, k, k_strides,
                    v, v_strides, o, o_strides, scale, mask, info, nullptr, nullptr, nullptr, stream);
}

splash_status splash_fwd_lse(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads, int q_len,
                             int kv_len, int head_dim, const void* q, const int64_t q_strides[3], const void* k,
                             const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* o,
                             const int64_t o_strides[3], float* lse, const int64_t lse_strides[2], float scale,
                             const splash_mask_desc* mask, const splash_mask_info* info, hipStream_t stream) {
  if (lse_strides == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse strides are null");
  return fwd_common(false, in_dtype, out_dtype, B, H, kv_heads, q_len, kv_len, head_dim, q, q_strides, k, k_strides,
                    v, v_strides, o, o_strides, scale, mask, info, nullptr, lse, lse_strides, stream);
}

splash_status splash_masked_fwd_lse(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                                    int q_len, int kv_len, int head_dim, const void* q, const int64_t q_strides[3],
                                    const void* k, const int64_t k_strides[3], const void* v,
                                    const int64_t v_strides[3], void* o, const int64_t o_strides[3], float* lse,
                                    const int64_t lse_strides[2], float scale, const splash_mask_desc* mask,
                                    const splash_mask_info* info, const splash_partial_masks* partial,
                                    hipStream_t stream) {
  if (lse_strides == nullptr) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "lse strides are null");
  return fwd_common(false, in_dtype, out_dtype, B, H, kv_heads, q_len, kv_len, head_dim, q, q_strides, k, k_strides,
                    v, v_strides, o, o_strides, scale, mask, info, partial, lse, lse_strides, stream);
}

splash_status splash_masked_bwd(int softmax, splash_dtype in_dtype, splash_dtype out_dtype, int B, int H,
                                int kv_heads, int q_len, int kv_len, int head_dim, const void* q,
                                const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                                const void* v, const int64_t v_strides[3], const void* d_o,
                                const int64_t do_strides[3], const float* lse, const float* delta,
                                const int64_t stat_strides[2], void* dq, const int64_t dq_strides[3], void* dk,
                                const int64_t dk_strides[3], void* dv, const int64_t dv_strides[3], float scale,
                                const splash_mask_desc* mask, const splash_mask_info* info,
                                const splash_partial_masks* partial, const splash_mask_info* info_dkv,
                                const splash_partial_masks* partial_dkv, hipStream_t stream) {
  if (softmax != 0 && softmax != 1)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "softmax=%d must be 0 or 1", softmax);
  return bwd_common(softmax == 1, in_dtype, out_dtype, B, H, kv_heads, q_len, kv_len, head_dim, q, q_strides, k,
                    k_strides, v, v_strides, d_o, do_strides, softmax == 1 ? lse : nullptr,
                    softmax == 1 ? delta : nullptr, softmax == 1 ? stat_strides : nullptr, dq, dq_strides, dk,
                    dk_strides, dv, dv_strides, scale, mask, info, info_dkv, stream, partial, partial_dkv);
}

splash_status splash_masked_fwd(int pointwise, splash_dtype in_dtype, splash_dtype out_dtype, int B, int H,
                                int kv_heads, int q_len, int kv_len, int head_dim, const void* q,
                                const int64_t q_strides[3], const void* k, const int64_t k_strides[3], const void* v,
                                const int64_t v_strides[3], void* o, const int64_t o_strides[3], float scale,
                                const splash_mask_desc* mask, const splash_mask_info* info,
                                const splash_partial_masks* partial, hipStream_t stream) {
  if (pointwise != 0 && pointwise != 1)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "pointwise=%d must be 0 or 1", pointwise);
  return fwd_common(pointwise == 1, in_dtype, out_dtype, B, H, kv_heads, q_len, kv_len, head_dim, q, q_strides, k,
                    k_strides, v, v_strides, o, o_strides, scale, mask, info, partial, nullptr, nullptr, stream);
}

}  // extern "C"
