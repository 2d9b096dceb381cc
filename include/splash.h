/*
 * splash.h — C ABI of the block-sparse masked attention forward library
 * (libsplash.so, AMD Instinct MI355X / gfx950).
 *
 * The operation is the forward pass of multi-head attention under a
 * block-sparse mask, computed block by block with an online softmax so that
 * the [S_q, S_kv] score matrix never exists:
 *   - "hstu_ops.py" (RecML recml/core/ops/hstu_ops.py): per-(head, q block,
 *     kv block) metadata read by `_next_nonzero` (a block runs when its class
 *     is > 0 and needs no element mask when it is not 1, and the kv block to
 *     fetch is `data_next`), element masks applied by `_apply_mask` (causal /
 *     local window / segment ids, ANDed), and the pointwise (SiLU, no softmax)
 *     forward `_pointwise_splash_attention_fwd_kernel_impl`;
 *   - "JAX 到 VLIW，以及 Pallas / Splash Attention 复习笔记": section 12
 *     (attention as softmax(Q Kᵀ) V), sections 15.1-15.3 (online softmax with
 *     running max m, denominator L and numerator O), section 18 (grid over
 *     (head, q block, kv block), kv axis sequential), section 21 (empty kv
 *     blocks are never loaded: indirection through data_next), section 23
 *     (only O is written back).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless marked HOST. Each call only enqueues
 *     work on `stream` (0 = the null stream) and never synchronizes.
 *   - All validation happens on the host before anything is enqueued. On any
 *     error nothing is enqueued, no output is touched, a status code is
 *     returned and splash_last_error() describes it. There is no fallback path.
 *   - The library allocates no device memory; the caller owns every buffer.
 *   - Positions: query q in [0, q_len), key k in [0, kv_len). Lengths need not
 *     be multiples of the block sizes: the last block of each axis is ragged
 *     and positions past the end are masked out.
 *   - Kernel choice: the softmax forwards at head_dim 128 with a band-only
 *     mask (no segment ids, no dense-mask store) and block_q 128 or 256 run a
 *     kernel with 64 query rows per wavefront when the problem has at least
 *     2048 of its 256-row workgroups, else the one-block kernel. The
 *     environment variable SPLASH_FWD_ROWS64=1 (or 0), read at each call,
 *     selects that kernel (or the other) whenever it applies. Both compute the
 *     same function with the same arithmetic per row.
 */
#ifndef SPLASH_H_
#define SPLASH_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPLASH_ABI_VERSION 1
#define SPLASH_MAX_MASK_HEADS 256

typedef enum {
  SPLASH_OK = 0,
  SPLASH_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad size/stride/alignment  */
  SPLASH_ERR_UNSUPPORTED = 2,       /* valid request without a compiled kernel */
  SPLASH_ERR_METADATA_MISMATCH = 3, /* metadata not built for this call        */
  SPLASH_ERR_HIP = 4                /* no device, or a HIP launch error        */
} splash_status;

typedef enum { SPLASH_F32 = 0, SPLASH_BF16 = 1 } splash_dtype;

/* Mask of one head ("hstu_ops.py", pointwise_splash_attention: CausalMask or
 * FullMask, optionally ANDed with LocalMask((w, w), offset=0)).
 * A pair (q, k) is allowed when
 *   (causal == 0 || k <= q) &&
 *   (window_left  < 0 || k >= q - window_left) &&
 *   (window_right < 0 || k <= q + window_right).
 * FULL = {0,-1,-1}; CAUSAL = {1,-1,-1}; causal AND local window w = {1,w,w}. */
typedef struct {
  int32_t causal;
  int32_t window_left;
  int32_t window_right;
} splash_head_mask;

/* Whole mask of a call. When segment ids are given, (q, k) is allowed only if
 * q_segment_ids[b, q] == kv_segment_ids[b, k] as well ("hstu_ops.py",
 * _apply_mask: segment equality ANDed with the other masks). */
typedef struct {
  int32_t num_mask_heads;          /* 1 (broadcast to every head) or H,
                                      at most SPLASH_MAX_MASK_HEADS          */
  const splash_head_mask* heads;   /* HOST array [num_mask_heads]           */
  const int32_t* q_segment_ids;    /* DEVICE int32 [B, q_len] row-major, or NULL */
  const int32_t* kv_segment_ids;   /* DEVICE int32 [B, kv_len] row-major, or NULL;
                                      both or neither                        */
} splash_mask_desc;

/* Block metadata. Shape [meta_batch, meta_heads, num_q_blocks, num_kv_blocks],
 * row-major, with meta_batch = B when segment ids are given (else 1),
 * meta_heads = num_mask_heads, num_q_blocks = ceil(q_len / block_q),
 * num_kv_blocks = ceil(kv_len / block_kv).
 *   block_mask[...,i,j]: 0 = no allowed pair in block (i, j) (never loaded),
 *                        1 = some pairs allowed (element mask applied),
 *                        2 = every pair of the whole block allowed (no mask).
 *   data_next[...,i,j]:  smallest j' >= j with block_mask[...,i,j'] != 0, or
 *                        num_kv_blocks if there is none.
 * The caller allocates both buffers (see splash_mask_info_entries) and fills
 * the six integer fields; splash_mask_info_build writes the two arrays. The
 * forward kernels read block_mask in aligned 32-bit words, so its allocation
 * must be 4-byte aligned and extend to a whole number of 32-bit words. */
typedef struct {
  int32_t meta_batch;
  int32_t meta_heads;
  int32_t num_q_blocks;
  int32_t num_kv_blocks;
  int32_t block_q;
  int32_t block_kv;
  int8_t* block_mask;   /* DEVICE int8  [meta_batch*meta_heads*nq*nk] */
  int32_t* data_next;   /* DEVICE int32 [meta_batch*meta_heads*nq*nk] */
} splash_mask_info;

/* Number of entries of each metadata array for this call (0 if the arguments
 * are invalid, or if a dimension is empty). Also usable to size the buffers:
 * block_mask needs that many bytes, data_next four times as many. Host only. */
size_t splash_mask_info_entries(int B, int H, int q_len, int kv_len, int block_q,
                                int block_kv, const splash_mask_desc* mask);

/* Build the block metadata on the GPU ("hstu_ops.py", _next_nonzero semantics;
 * study notes section 21, data_next).
 * block_q, block_kv: positive, at most 1024. `info` must describe buffers of
 * the shape given above; its integer fields are checked against the call.
 * Segment ids are read on the device; with segment ids the build first uses
 * data_next as its own scratch (per-block runs of equal ids) and then
 * overwrites it with the result, so data_next must not be read by other work
 * until the call's kernels have finished on `stream`. Errors: INVALID_ARGUMENT (bad sizes,
 * null pointers, one segment array without the other, info shape wrong),
 * HIP (launch failure / no device). */
splash_status splash_mask_info_build(int B, int H, int q_len, int kv_len, int block_q,
                                     int block_kv, const splash_mask_desc* mask,
                                     const splash_mask_info* info, hipStream_t stream);

/* Softmax attention forward:
 *   o[b,h,q,:] = sum_{k allowed} e^{s_k - m} v[b,h,k,:] / sum_{k allowed} e^{s_k - m}
 * with s_k = scale * <q[b,h,q,:], k[b,h,k,:]>, m the row max over allowed keys;
 * a row with no allowed key is written as 0. Empty blocks (block_mask 0) are
 * skipped through data_next and never read; the element mask is evaluated only
 * on blocks of class 1 (study notes sections 15, 18, 21, 23).
 *
 * Tensors: q [B, H, q_len, head_dim], k and v [B, H, kv_len, head_dim],
 * o [B, H, q_len, head_dim]. `*_strides` give the element strides of the
 * batch, head and sequence axes (int64, HOST arrays of 3); head_dim is
 * contiguous. This covers both [B,H,S,D] and the [B,S,H,D] layout of
 * "hstu_ops.py" pointwise_splash_attention without copies. Every row must
 * start 16-byte aligned (base pointers and strides accordingly), and
 * consecutive rows of a tensor must lie less than 64 MiB apart
 * (UNSUPPORTED otherwise; the same holds for every tensor of the backward
 * entry points).
 *
 * Supported: in_dtype/out_dtype F32/F32, BF16/BF16 or BF16/F32; head_dim 64 or
 * 128; block_q in {64, 128, 256} and block_kv in {64, 128}. Arithmetic: F32 inputs are computed
 * in fp32; BF16 inputs use bf16 matrix cores with fp32 accumulation and fp32
 * softmax statistics, and the probabilities are rounded to bf16 for P·V.
 * `info` must have been built for the same B, H, lengths, block sizes, mask
 * heads and segment-id presence (METADATA_MISMATCH otherwise). */
splash_status splash_fwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H,
                         int q_len, int kv_len, int head_dim,
                         const void* q, const int64_t q_strides[3],
                         const void* k, const int64_t k_strides[3],
                         const void* v, const int64_t v_strides[3],
                         void* o, const int64_t o_strides[3],
                         float scale, const splash_mask_desc* mask,
                         const splash_mask_info* info, hipStream_t stream);

/* Pointwise (HSTU) attention forward, "hstu_ops.py",
 * _pointwise_splash_attention_fwd_kernel_impl:
 *   o[b,h,q,:] = (1/q_len) * sum_{k allowed} silu(s_k) v[b,h,k,:],
 *   silu(x) = x / (1 + e^{-x}), s_k as above.
 * The contributions of all kv blocks are summed (the page's per-slice
 * overwrite of the output is read as this accumulation). Same arguments,
 * layouts, support matrix and errors as splash_fwd. */
splash_status splash_pointwise_fwd(splash_dtype in_dtype, splash_dtype out_dtype, int B,
                                   int H, int q_len, int kv_len, int head_dim,
                                   const void* q, const int64_t q_strides[3],
                                   const void* k, const int64_t k_strides[3],
                                   const void* v, const int64_t v_strides[3],
                                   void* o, const int64_t o_strides[3],
                                   float scale, const splash_mask_desc* mask,
                                   const splash_mask_info* info, hipStream_t stream);

/* Grouped-query (and multi-query) forms of the two forwards ("JAX 到 VLIW ..."
 * study notes, section 21: several query heads share one K/V head, and query
 * head h reads K/V head h / (H / kv_heads)). Same arguments, layouts, support
 * matrix and errors as splash_fwd / splash_pointwise_fwd, except that k and v
 * are [B, kv_heads, kv_len, head_dim] (their head stride steps over K/V
 * heads). kv_heads must divide H (INVALID_ARGUMENT otherwise); kv_heads == H
 * is plain multi-head attention and kv_heads == 1 multi-query attention. The
 * mask heads and the metadata stay per query head. */
splash_status splash_gqa_fwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                             int q_len, int kv_len, int head_dim,
                             const void* q, const int64_t q_strides[3],
                             const void* k, const int64_t k_strides[3],
                             const void* v, const int64_t v_strides[3],
                             void* o, const int64_t o_strides[3],
                             float scale, const splash_mask_desc* mask,
                             const splash_mask_info* info, hipStream_t stream);
splash_status splash_gqa_pointwise_fwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H,
                                       int kv_heads, int q_len, int kv_len, int head_dim,
                                       const void* q, const int64_t q_strides[3],
                                       const void* k, const int64_t k_strides[3],
                                       const void* v, const int64_t v_strides[3],
                                       void* o, const int64_t o_strides[3],
                                       float scale, const splash_mask_desc* mask,
                                       const splash_mask_info* info, hipStream_t stream);

/* Dense masks ("hstu_ops.py", pointwise_splash_attention: a numpy array mask
 * of shape (q_len, kv_len) becomes a NumpyMask, ANDed with the local window;
 * the forward fetches the mask of a partial block through a second index map,
 * mask_next, into a store of mask blocks, so equal partial blocks share one
 * entry).
 *
 * splash_dense_mask_info_host builds, on the host, the metadata of the mask
 *   allowed(h, q, k) = dense[h', q, k] != 0 AND the band of head mask h'',
 * with h' = 0 if dense_heads == 1 else h, h'' likewise for num_mask_heads,
 * for meta_heads = max(dense_heads, num_mask_heads) metadata heads (each count
 * 1 or meta_heads), meta_batch 1 (no segment ids). ALL POINTERS ARE HOST.
 *   dense:       [dense_heads, q_len, kv_len] bytes, nonzero = allowed.
 *   block_mask, data_next: as splash_mask_info, [meta_heads, nq, nk].
 *   mask_next:   [meta_heads, nq, nk]: for a block of class 1, its entry of
 *                mask_blocks; 0 for the other blocks.
 *   mask_blocks: [capacity, block_q, block_kv / 32] uint32: row r of an
 *                entry is block_kv / 32 words, bit b of word w standing for
 *                key offset 32 w + b of the block; positions past the
 *                sequence ends are 0. Equal partial blocks share an entry.
 *   num_blocks:  out: the number of entries the mask needs.
 * With block_mask, data_next and mask_next all NULL the call only sets
 * *num_blocks (size the store with it). Otherwise capacity must be at least
 * *num_blocks (INVALID_ARGUMENT, and nothing written, if not). block_kv must be
 * a multiple of 32. The caller copies the arrays to the device for
 * splash_masked_fwd. This call runs on the calling thread and touches no GPU. */
splash_status splash_dense_mask_info_host(int q_len, int kv_len, int block_q, int block_kv,
                                          int num_mask_heads, const splash_head_mask* heads,
                                          int dense_heads, const uint8_t* dense, int meta_heads,
                                          int8_t* block_mask, int32_t* data_next, int32_t* mask_next,
                                          uint32_t* mask_blocks, int64_t capacity, int64_t* num_blocks);

/* The same with segment ids and either metadata layout: for B batch rows,
 *   allowed(b, h, q, k) = dense[h', q, k] != 0 AND the band of head mask h''
 *                         AND q_segment_ids[b, q] == kv_segment_ids[b, k]
 * ("hstu_ops.py", _apply_mask: the stored mask block, the mask function and
 * segment equality, ANDed). q_segment_ids [B, q_len] and kv_segment_ids
 * [B, kv_len] are HOST int32 arrays, both or neither. With them the metadata
 * has meta_batch = B (every array gains a leading batch axis; the store is
 * shared by all batch rows); without them meta_batch = 1 (B is then only
 * range-checked). columns = 0 gives the row layout above (for the forward and the
 * backward's dQ walk); columns = 1 the dK/dV walk's layout of
 * splash_mask_info_build_dkv: block_mask, data_next and mask_next are
 * [meta_batch, meta_heads, nk, nq], data_next running along q blocks ("hstu_ops.py"
 * builds the backward's dK/dV mask blocks separately, bwd_mask_info). The
 * store entries are [block_q, block_kv / 32] words either way. Everything
 * else (sizing with a count-only call, capacity, errors) as
 * splash_dense_mask_info_host, which is this call with B = 1, no segment ids
 * and columns = 0. ALL POINTERS ARE HOST. */
splash_status splash_dense_mask_info_host_ex(int B, int q_len, int kv_len, int block_q, int block_kv,
                                             int num_mask_heads, const splash_head_mask* heads,
                                             int dense_heads, const uint8_t* dense, int meta_heads,
                                             const int32_t* q_segment_ids, const int32_t* kv_segment_ids,
                                             int columns, int8_t* block_mask, int32_t* data_next,
                                             int32_t* mask_next, uint32_t* mask_blocks, int64_t capacity,
                                             int64_t* num_blocks);

/* Device copies of a dense mask's partial blocks (see above). */
typedef struct {
  const int32_t* mask_next;     /* DEVICE, the layout of its metadata's block_mask */
  const uint32_t* mask_blocks;  /* DEVICE [num_blocks, block_q, block_kv / 32]     */
  int64_t num_blocks;
} splash_partial_masks;

/* General forward: pointwise = 0 is splash_fwd, 1 is splash_pointwise_fwd,
 * with grouped-query K/V (kv_heads, as splash_gqa_fwd) and optional dense-mask
 * blocks. With partial == NULL this is exactly those calls. With partial
 * given, `info` holds the block_mask / data_next of the same dense mask (its
 * meta_heads 1 or H, the head masks 1 or as many), and on every block of
 * class 1 the block's bits are ANDed with the head band. Segment ids may be
 * given with a dense mask: the metadata must then come from
 * splash_dense_mask_info_host_ex with the same ids (meta_batch = B), which
 * folds segment equality into the classes and bits, so the kernel does not
 * read the device ids (METADATA_MISMATCH if meta_batch is not B; with B = 1
 * the library cannot tell metadata built without the ids). mask_next entries
 * outside [0, num_blocks) are clamped, so no metadata content makes the
 * kernel read outside the store. */
splash_status splash_masked_fwd(int pointwise, splash_dtype in_dtype, splash_dtype out_dtype, int B, int H,
                                int kv_heads, int q_len, int kv_len, int head_dim,
                                const void* q, const int64_t q_strides[3],
                                const void* k, const int64_t k_strides[3],
                                const void* v, const int64_t v_strides[3],
                                void* o, const int64_t o_strides[3],
                                float scale, const splash_mask_desc* mask,
                                const splash_mask_info* info, const splash_partial_masks* partial,
                                hipStream_t stream);

/* ---- Pointwise backward ----
 *
 * "hstu_ops.py" (RecML), _pointwise_splash_attention_bwd_kernel_impl and
 * _pointwise_splash_attention_bwd_kernel: the gradients of
 * splash_pointwise_fwd. With x = scale q·k, sig = logistic(x) (0 where the
 * mask forbids the pair) and dO the gradient of the output:
 *   p  = x sig / q_len,                     dV_k = sum_q p dO_q
 *   ds = (dO_q·v_k) sig (1 + x (1 - sig)) / q_len
 *   dK_k = scale sum_q ds q_q,              dQ_q = scale sum_k ds k_k
 * dQ is computed over the row walk (metadata of splash_mask_info_build), dK
 * and dV over the column walk that the page's dK/dV grid uses (metadata of
 * splash_mask_info_build_dkv, possibly with other block sizes). */

/* Metadata of the dK/dV pass, stored by columns: both arrays are
 * [meta_batch, meta_heads, nk, nq] (info's num_q_blocks and num_kv_blocks
 * still give nq and nk). block_mask[.., j, i] is the class that
 * splash_mask_info_build gives block (i, j), and data_next[.., j, i] = the
 * first q block i' >= i of kv-block column j whose class is not 0, else nq
 * (_next_nonzero with next_i=True reads data_next[h, i, j] as the q block to
 * fetch; the column layout keeps each column's walk in consecutive memory).
 * Same arguments, checks and errors as splash_mask_info_build; enqueued on
 * `stream`. */
splash_status splash_mask_info_build_dkv(int B, int H, int q_len, int kv_len, int block_q, int block_kv,
                                         const splash_mask_desc* mask, const splash_mask_info* info,
                                         hipStream_t stream);

/* dq [B, H, q_len, D], dk and dv [B, kv_heads, kv_len, D] from q, k, v and
 * d_o ([B, H, q_len, D], the output gradient), for the mask `mask`.
 * Strides, dtypes (f32 -> f32, bf16 -> bf16, bf16 -> f32: the gradients take
 * out_dtype), head_dim (64, 128) and kv_heads (a divisor of H; query head h
 * reads K/V head h / (H / kv_heads), and a K/V head's gradients sum over its
 * query heads) are as for splash_gqa_pointwise_fwd. `info` (row walk) must
 * come from splash_mask_info_build with block_q in {64, 128, 256} and
 * block_kv in {64, 128}; `info_dkv` (column walk) from
 * splash_mask_info_build_dkv with block_q a multiple of 32 in [32, 1024] and
 * block_kv in {64, 128}. Both for this call's shapes, mask heads and
 * segment ids (METADATA_MISMATCH otherwise). dq, dk and dv are fully
 * overwritten (0 for rows no pair reaches); inputs are read only; the output
 * buffers must not overlap the inputs or each other. Enqueued on `stream`. */
splash_status splash_pointwise_bwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                                   int q_len, int kv_len, int head_dim,
                                   const void* q, const int64_t q_strides[3],
                                   const void* k, const int64_t k_strides[3],
                                   const void* v, const int64_t v_strides[3],
                                   const void* d_o, const int64_t do_strides[3],
                                   void* dq, const int64_t dq_strides[3],
                                   void* dk, const int64_t dk_strides[3],
                                   void* dv, const int64_t dv_strides[3],
                                   float scale, const splash_mask_desc* mask,
                                   const splash_mask_info* info, const splash_mask_info* info_dkv,
                                   hipStream_t stream);

/* ---- Softmax log-sum-exp and backward ----
 *
 * The study notes "JAX 到 VLIW ..." give the softmax forward (sections 12 and
 * 15); "hstu_ops.py" gives, for the pointwise variant, the custom_vjp pattern
 * in which the forward hands the backward its residuals. The softmax
 * backward here is the gradient of the softmax definition with the
 * forward's per-row log-sum-exp as the residual: with x = scale q·k,
 *   LSE_q = log sum_k e^{x_qk} (allowed keys; -inf for a row with none),
 *   P = e^{x - LSE} (0 where masked),  delta_q = dO_q · O_q,
 *   dV = Pᵀ dO,  dS = P (dO Vᵀ - delta),  dQ = scale dS K,  dK = scale dSᵀ Q. */

/* splash_gqa_fwd (softmax) that also writes lse[b * lse_strides[0] +
 * h * lse_strides[1] + i] = LSE of row i (fp32, rows contiguous, caller
 * owned, 4-byte aligned). Same arguments, checks and errors otherwise. */
splash_status splash_fwd_lse(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads, int q_len,
                             int kv_len, int head_dim,
                             const void* q, const int64_t q_strides[3],
                             const void* k, const int64_t k_strides[3],
                             const void* v, const int64_t v_strides[3],
                             void* o, const int64_t o_strides[3],
                             float* lse, const int64_t lse_strides[2],
                             float scale, const splash_mask_desc* mask, const splash_mask_info* info,
                             hipStream_t stream);

/* delta[b * delta_strides[0] + h * delta_strides[1] + i] = sum_d o[b,h,i,d] *
 * d_o[b,h,i,d] in fp32, for o and d_o [B, H, q_len, head_dim] of `dtype`
 * (strided as the forward's tensors). The caller owns delta (fp32,
 * 4-byte aligned). Enqueued on `stream`. */
splash_status splash_softmax_bwd_preprocess(splash_dtype dtype, int B, int H, int q_len, int head_dim,
                                            const void* o, const int64_t o_strides[3],
                                            const void* d_o, const int64_t do_strides[3],
                                            float* delta, const int64_t delta_strides[2], hipStream_t stream);

/* dq, dk, dv of softmax attention (splash_gqa_fwd) from q, k, v, d_o and the
 * forward's lse and the preprocess's delta (both fp32, indexed as
 * b * stat_strides[0] + h * stat_strides[1] + i). Everything else (dtypes,
 * head_dim, kv_heads, the two metadata structs, block sizes, overwriting and
 * errors) is as for splash_pointwise_bwd. */
splash_status splash_softmax_bwd(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                                 int q_len, int kv_len, int head_dim,
                                 const void* q, const int64_t q_strides[3],
                                 const void* k, const int64_t k_strides[3],
                                 const void* v, const int64_t v_strides[3],
                                 const void* d_o, const int64_t do_strides[3],
                                 const float* lse, const float* delta, const int64_t stat_strides[2],
                                 void* dq, const int64_t dq_strides[3],
                                 void* dk, const int64_t dk_strides[3],
                                 void* dv, const int64_t dv_strides[3],
                                 float scale, const splash_mask_desc* mask,
                                 const splash_mask_info* info, const splash_mask_info* info_dkv,
                                 hipStream_t stream);

/* Softmax forward with the per-row log-sum-exp (as splash_fwd_lse) under a
 * dense mask (as splash_masked_fwd with pointwise = 0): the residuals of the
 * softmax backward for a dense-mask model. partial may be NULL. */
splash_status splash_masked_fwd_lse(splash_dtype in_dtype, splash_dtype out_dtype, int B, int H, int kv_heads,
                                    int q_len, int kv_len, int head_dim,
                                    const void* q, const int64_t q_strides[3],
                                    const void* k, const int64_t k_strides[3],
                                    const void* v, const int64_t v_strides[3],
                                    void* o, const int64_t o_strides[3],
                                    float* lse, const int64_t lse_strides[2],
                                    float scale, const splash_mask_desc* mask, const splash_mask_info* info,
                                    const splash_partial_masks* partial, hipStream_t stream);

/* General backward: softmax = 0 is splash_pointwise_bwd (lse, delta and
 * stat_strides are ignored), 1 is splash_softmax_bwd, with optional dense
 * masks ("hstu_ops.py", _pointwise_splash_attention_bwd: the dQ and dK/dV
 * kernels fetch a partial block's mask through their own mask_next into
 * their own store of mask blocks, built for their own block sizes). partial
 * and partial_dkv are both NULL (exactly the calls above) or both given:
 * `info` and `partial` from splash_dense_mask_info_host_ex with columns = 0,
 * `info_dkv` and `partial_dkv` with columns = 1, both for the same mask and
 * segment ids (as for splash_masked_fwd, the ids are then folded into the
 * metadata and not read on the device) and the same metadata heads (1 or H);
 * block_kv of both walks in {64, 128}. Errors as for the two calls above,
 * plus INVALID_ARGUMENT for one of the two dense structs missing, null or
 * misaligned arrays. */
splash_status splash_masked_bwd(int softmax, splash_dtype in_dtype, splash_dtype out_dtype, int B, int H,
                                int kv_heads, int q_len, int kv_len, int head_dim,
                                const void* q, const int64_t q_strides[3],
                                const void* k, const int64_t k_strides[3],
                                const void* v, const int64_t v_strides[3],
                                const void* d_o, const int64_t do_strides[3],
                                const float* lse, const float* delta, const int64_t stat_strides[2],
                                void* dq, const int64_t dq_strides[3],
                                void* dk, const int64_t dk_strides[3],
                                void* dv, const int64_t dv_strides[3],
                                float scale, const splash_mask_desc* mask,
                                const splash_mask_info* info, const splash_partial_masks* partial,
                                const splash_mask_info* info_dkv, const splash_partial_masks* partial_dkv,
                                hipStream_t stream);

/* Static name of a status code. */
const char* splash_status_string(splash_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* splash_last_error(void);
/* SPLASH_ABI_VERSION of the loaded library. */
int splash_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLASH_H_ */
