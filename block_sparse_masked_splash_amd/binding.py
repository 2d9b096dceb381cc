"""ctypes binding of libsplash.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
turns torch tensors into device pointers, strides and the caller's stream,
and turns status codes into exceptions. It has no fallback: if the library
is missing or a call fails, it raises.
"""

from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsplash.so")

SPLASH_OK = 0
SPLASH_ERR_INVALID_ARGUMENT = 1
SPLASH_ERR_UNSUPPORTED = 2
SPLASH_ERR_METADATA_MISMATCH = 3
SPLASH_ERR_HIP = 4
SPLASH_F32 = 0
SPLASH_BF16 = 1
MAX_MASK_HEADS = 256

# Exported symbols, as declared in include/splash.h.
SYMBOLS = (
    "splash_mask_info_entries",
    "splash_mask_info_build",
    "splash_fwd",
    "splash_pointwise_fwd",
    "splash_gqa_fwd",
    "splash_gqa_pointwise_fwd",
    "splash_dense_mask_info_host",
    "splash_masked_fwd",
    "splash_mask_info_build_dkv",
    "splash_pointwise_bwd",
    "splash_fwd_lse",
    "splash_softmax_bwd_preprocess",
    "splash_softmax_bwd",
    "splash_dense_mask_info_host_ex",
    "splash_masked_fwd_lse",
    "splash_masked_bwd",
    "splash_status_string",
    "splash_last_error",
    "splash_abi_version",
)


class SplashError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class HeadMaskC(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32)]


class MaskDescC(ctypes.Structure):
    _fields_ = [("num_mask_heads", ctypes.c_int32), ("heads", ctypes.POINTER(HeadMaskC)),
                ("q_segment_ids", ctypes.c_void_p), ("kv_segment_ids", ctypes.c_void_p)]


class MaskInfoC(ctypes.Structure):
    _fields_ = [("meta_batch", ctypes.c_int32), ("meta_heads", ctypes.c_int32),
                ("num_q_blocks", ctypes.c_int32), ("num_kv_blocks", ctypes.c_int32),
                ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32),
                ("block_mask", ctypes.c_void_p), ("data_next", ctypes.c_void_p)]


class PartialMasksC(ctypes.Structure):
    _fields_ = [("mask_next", ctypes.c_void_p), ("mask_blocks", ctypes.c_void_p), ("num_blocks", ctypes.c_int64)]


_I64x3 = ctypes.c_int64 * 3
_FWD_ARGS = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
             ctypes.c_int,
             ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
             ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
             ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
             ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
             ctypes.c_float, ctypes.POINTER(MaskDescC), ctypes.POINTER(MaskInfoC), ctypes.c_void_p]
# grouped-query forms: kv_heads follows H
_GQA_ARGS = _FWD_ARGS[:4] + [ctypes.c_int] + _FWD_ARGS[4:]
# general form: pointwise flag first, partial masks before the stream
_MASKED_ARGS = [ctypes.c_int] + _GQA_ARGS[:-1] + [ctypes.POINTER(PartialMasksC), ctypes.c_void_p]
_T = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
_BWD_ARGS = ([ctypes.c_int] * 8 + _T * 7
             + [ctypes.c_float, ctypes.POINTER(MaskDescC), ctypes.POINTER(MaskInfoC), ctypes.POINTER(MaskInfoC),
                ctypes.c_void_p])
_I64p = ctypes.POINTER(ctypes.c_int64)
_SM_BWD_ARGS = ([ctypes.c_int] * 8 + _T * 4 + [ctypes.c_void_p, ctypes.c_void_p, _I64p] + _T * 3
                + [ctypes.c_float, ctypes.POINTER(MaskDescC), ctypes.POINTER(MaskInfoC), ctypes.POINTER(MaskInfoC),
                   ctypes.c_void_p])
_LSE_ARGS = ([ctypes.c_int] * 8 + _T * 4 + [ctypes.c_void_p, _I64p]
             + [ctypes.c_float, ctypes.POINTER(MaskDescC), ctypes.POINTER(MaskInfoC), ctypes.c_void_p])
# dense-mask forms: partial masks after the metadata they go with
_MASKED_LSE_ARGS = _LSE_ARGS[:-1] + [ctypes.POINTER(PartialMasksC), ctypes.c_void_p]
_MASKED_BWD_ARGS = ([ctypes.c_int] * 9 + _T * 4 + [ctypes.c_void_p, ctypes.c_void_p, _I64p] + _T * 3
                    + [ctypes.c_float, ctypes.POINTER(MaskDescC), ctypes.POINTER(MaskInfoC),
                       ctypes.POINTER(PartialMasksC), ctypes.POINTER(MaskInfoC), ctypes.POINTER(PartialMasksC),
                       ctypes.c_void_p])
_I64x2 = ctypes.c_int64 * 2

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsplash.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_masked_splash_amd.build` "
            "(there is no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    lib.splash_mask_info_entries.restype = ctypes.c_size_t
    lib.splash_mask_info_entries.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(MaskDescC)]
    for name in ("splash_mask_info_build", "splash_mask_info_build_dkv"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(MaskDescC), ctypes.POINTER(MaskInfoC), ctypes.c_void_p]
    lib.splash_pointwise_bwd.restype = ctypes.c_int
    lib.splash_pointwise_bwd.argtypes = _BWD_ARGS
    lib.splash_softmax_bwd.restype = ctypes.c_int
    lib.splash_softmax_bwd.argtypes = _SM_BWD_ARGS
    lib.splash_fwd_lse.restype = ctypes.c_int
    lib.splash_fwd_lse.argtypes = _LSE_ARGS
    lib.splash_softmax_bwd_preprocess.restype = ctypes.c_int
    lib.splash_softmax_bwd_preprocess.argtypes = [ctypes.c_int] * 5 + _T * 2 + [ctypes.c_void_p, _I64p,
                                                                                ctypes.c_void_p]
    for name in ("splash_fwd", "splash_pointwise_fwd"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = _FWD_ARGS
    for name in ("splash_gqa_fwd", "splash_gqa_pointwise_fwd"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = _GQA_ARGS
    lib.splash_masked_fwd.restype = ctypes.c_int
    lib.splash_masked_fwd.argtypes = _MASKED_ARGS
    lib.splash_dense_mask_info_host.restype = ctypes.c_int
    lib.splash_dense_mask_info_host.argtypes = (
        [ctypes.c_int] * 5 + [ctypes.POINTER(HeadMaskC), ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        + [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)])
    lib.splash_dense_mask_info_host_ex.restype = ctypes.c_int
    lib.splash_dense_mask_info_host_ex.argtypes = (
        [ctypes.c_int] * 6 + [ctypes.POINTER(HeadMaskC), ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        + [ctypes.c_void_p] * 2 + [ctypes.c_int] + [ctypes.c_void_p] * 4
        + [ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)])
    lib.splash_masked_fwd_lse.restype = ctypes.c_int
    lib.splash_masked_fwd_lse.argtypes = _MASKED_LSE_ARGS
    lib.splash_masked_bwd.restype = ctypes.c_int
    lib.splash_masked_bwd.argtypes = _MASKED_BWD_ARGS
    lib.splash_status_string.restype = ctypes.c_char_p
    lib.splash_status_string.argtypes = [ctypes.c_int]
    lib.splash_last_error.restype = ctypes.c_char_p
    lib.splash_last_error.argtypes = []
    lib.splash_abi_version.restype = ctypes.c_int
    lib.splash_abi_version.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != SPLASH_OK:
        msg = load_library().splash_last_error().decode()
        raise SplashError(status, msg)


# ---------------------------------------------------------------------------
# masks and metadata
# ---------------------------------------------------------------------------


def _head_array(head_masks):
    hm = [tuple(int(x) for x in m) for m in head_masks]
    arr = (HeadMaskC * max(1, len(hm)))()
    for n, (c, wl, wr) in enumerate(hm):
        arr[n] = HeadMaskC(c, wl, wr)
    return arr, len(hm)


def _seg_ptr(t, B, S, name):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.device.type != "cuda" or tuple(t.shape) != (B, S) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor of shape {(B, S)}")
    return t.data_ptr()


@dataclasses.dataclass
class MaskInfo:
    """Block metadata on the GPU plus the mask it was built from."""
    B: int
    H: int
    q_len: int
    kv_len: int
    block_q: int
    block_kv: int
    head_masks: tuple
    q_segment_ids: torch.Tensor | None
    kv_segment_ids: torch.Tensor | None
    block_mask: torch.Tensor   # int8 [meta_batch, meta_heads, nq, nk]
    data_next: torch.Tensor    # int32, same shape
    # dense masks only: mask_next int32 (same shape) and the store of partial
    # blocks, int32 [num_blocks, block_q, block_kv // 32] (bits, see splash.h)
    mask_next: torch.Tensor | None = None
    mask_blocks: torch.Tensor | None = None
    # dK/dV metadata: block_mask and data_next are [meta_batch, meta_heads, nk, nq]
    columns: bool = False

    @property
    def dense(self) -> bool:
        return self.mask_next is not None

    def partial_struct(self):
        n = 0 if self.mask_blocks is None else self.mask_blocks.shape[0]
        return PartialMasksC(self.mask_next.data_ptr() if self.mask_next.numel() else None,
                             self.mask_blocks.data_ptr() if n else None, n)

    def mask_desc(self):
        arr, n = _head_array(self.head_masks)
        desc = MaskDescC(n, ctypes.cast(arr, ctypes.POINTER(HeadMaskC)),
                         _seg_ptr(self.q_segment_ids, self.B, self.q_len, "q_segment_ids"),
                         _seg_ptr(self.kv_segment_ids, self.B, self.kv_len, "kv_segment_ids"))
        return desc, arr

    def info_struct(self):
        Bm, Hm, nq, nk = self.block_mask.shape
        if self.columns:
            nq, nk = nk, nq
        return MaskInfoC(Bm, Hm, nq, nk, self.block_q, self.block_kv,
                         self.block_mask.data_ptr() if self.block_mask.numel() else None,
                         self.data_next.data_ptr() if self.data_next.numel() else None)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def dense_mask_info_build(B: int, H: int, dense, head_masks=((0, -1, -1),), block_q: int = 128,
                          block_kv: int = 128, device="cuda", q_segment_ids=None, kv_segment_ids=None,
                          columns: bool = False) -> MaskInfo:
    """Metadata of an arbitrary dense mask ANDed with head masks (and, with
    segment ids, with segment equality), built on the host by the library and
    copied to ``device``.

    ``dense``: boolean [q_len, kv_len] (shared by all heads) or [H, q_len,
    kv_len]; ``head_masks``: 1 or H (causal, window_left, window_right)
    triples; segment ids: int32 [B, q_len] and [B, kv_len] (CPU or GPU),
    folded into the metadata (one metadata batch row per batch row).
    ``columns``: the layout of the backward's dK/dV walk (as
    ``mask_info_build_dkv``) instead of the row walk."""
    lib = load_library()
    d = torch.as_tensor(dense).to("cpu")
    if d.dim() == 2:
        d = d.unsqueeze(0)
    if d.dim() != 3 or d.shape[0] not in (1, H):
        raise ValueError("dense must be [q_len, kv_len] or [H, q_len, kv_len]")
    d = d.to(torch.uint8).contiguous()
    Hd, q_len, kv_len = d.shape
    head_masks = tuple(tuple(int(x) for x in m) for m in head_masks)
    if len(head_masks) not in (1, H) or len(head_masks) > MAX_MASK_HEADS:
        raise ValueError("head_masks must hold 1 or H entries")
    if (q_segment_ids is None) != (kv_segment_ids is None):
        raise ValueError("both or neither of q_segment_ids and kv_segment_ids must be given")
    seg = q_segment_ids is not None
    if seg:
        qs_h = torch.as_tensor(q_segment_ids).to("cpu", torch.int32).contiguous()
        ks_h = torch.as_tensor(kv_segment_ids).to("cpu", torch.int32).contiguous()
        if tuple(qs_h.shape) != (B, q_len) or tuple(ks_h.shape) != (B, kv_len):
            raise ValueError(f"segment ids must be [B, q_len] = {(B, q_len)} and [B, kv_len] = {(B, kv_len)}")
    Hm = max(Hd, len(head_masks))
    Bm = B if seg else 1
    nq = -(-q_len // block_q) if block_q > 0 else 0
    nk = -(-kv_len // block_kv) if block_kv > 0 else 0
    arr, nmh = _head_array(head_masks)
    heads_p = ctypes.cast(arr, ctypes.POINTER(HeadMaskC))
    qs_p = qs_h.data_ptr() if seg else None
    ks_p = ks_h.data_ptr() if seg else None
    count = ctypes.c_int64(0)
    st = lib.splash_dense_mask_info_host_ex(B, q_len, kv_len, block_q, block_kv, nmh, heads_p, Hd, d.data_ptr(), Hm,
                                            qs_p, ks_p, int(columns), None, None, None, None, 0, ctypes.byref(count))
    _check(st)
    n = count.value
    shape = (Bm, Hm, nk, nq) if columns else (Bm, Hm, nq, nk)
    entries = Bm * Hm * nq * nk
    bmask = torch.empty((entries + 3) // 4 * 4, dtype=torch.int8)
    dnext = torch.empty(shape, dtype=torch.int32)
    mnext = torch.empty(shape, dtype=torch.int32)
    wpr = block_kv // 32
    blocks = torch.empty((n, block_q, wpr), dtype=torch.int32)
    st = lib.splash_dense_mask_info_host_ex(B, q_len, kv_len, block_q, block_kv, nmh, heads_p, Hd, d.data_ptr(), Hm,
                                            qs_p, ks_p, int(columns), bmask.data_ptr(), dnext.data_ptr(),
                                            mnext.data_ptr(), blocks.data_ptr() if n else None, n,
                                            ctypes.byref(count))
    _check(st)
    device = torch.device(device)
    bmask_dev = bmask.to(device)[:entries].view(shape)
    qs_d = qs_h.to(device) if seg else None
    ks_d = ks_h.to(device) if seg else None
    return MaskInfo(B, H, q_len, kv_len, block_q, block_kv, head_masks, qs_d, ks_d, bmask_dev,
                    dnext.to(device), mnext.to(device), blocks.to(device), columns=bool(columns))


def dense_mask_info_build_dkv(B: int, H: int, dense, head_masks=((0, -1, -1),), block_q: int = 128,
                              block_kv: int = 128, device="cuda", q_segment_ids=None,
                              kv_segment_ids=None) -> MaskInfo:
    """``dense_mask_info_build`` in the layout of the backward's dK/dV walk."""
    return dense_mask_info_build(B, H, dense, head_masks, block_q, block_kv, device, q_segment_ids,
                                 kv_segment_ids, columns=True)


def mask_info_build(B: int, H: int, q_len: int, kv_len: int, head_masks, block_q: int = 128,
                    block_kv: int = 128, q_segment_ids=None, kv_segment_ids=None,
                    device="cuda", out: MaskInfo | None = None) -> MaskInfo:
    """Build block metadata with the library's kernel on the current stream.

    ``head_masks``: one (causal, window_left, window_right) triple for every
    head, or a single one broadcast to all heads. ``out`` reuses the buffers of
    an earlier MaskInfo of the same shape."""
    return _mask_info(False, B, H, q_len, kv_len, head_masks, block_q, block_kv, q_segment_ids, kv_segment_ids,
                      device, out)


def mask_info_build_dkv(B: int, H: int, q_len: int, kv_len: int, head_masks, block_q: int = 128,
                        block_kv: int = 128, q_segment_ids=None, kv_segment_ids=None,
                        device="cuda", out: MaskInfo | None = None) -> MaskInfo:
    """Metadata of the backward's dK/dV pass, stored by columns: block_mask
    and data_next are [meta_batch, meta_heads, nk, nq]; the same block
    classes, with ``data_next`` walking each kv-block column over q blocks."""
    return _mask_info(True, B, H, q_len, kv_len, head_masks, block_q, block_kv, q_segment_ids, kv_segment_ids,
                      device, out)


def _mask_info(dkv: bool, B, H, q_len, kv_len, head_masks, block_q, block_kv, q_segment_ids, kv_segment_ids,
               device, out) -> MaskInfo:
    lib = load_library()
    device = torch.device(device)
    head_masks = tuple(tuple(int(x) for x in m) for m in head_masks)
    if len(head_masks) not in (1, H) or len(head_masks) > MAX_MASK_HEADS:
        raise ValueError("head_masks must hold 1 or H entries")
    if (q_segment_ids is None) != (kv_segment_ids is None):
        raise ValueError("both or neither of q_segment_ids and kv_segment_ids must be given")
    Bm = B if q_segment_ids is not None else 1
    nq = -(-q_len // block_q) if block_q > 0 else 0
    nk = -(-kv_len // block_kv) if block_kv > 0 else 0
    shape = (Bm, len(head_masks), nk, nq) if dkv else (Bm, len(head_masks), nq, nk)
    if out is not None and tuple(out.block_mask.shape) == shape:
        bmask, dnext = out.block_mask, out.data_next
    else:
        n = shape[0] * shape[1] * shape[2] * shape[3]
        # the kernels read block classes as aligned 32-bit words: pad to whole words
        bmask = torch.empty((n + 3) // 4 * 4, dtype=torch.int8, device=device)[:n].view(shape)
        dnext = torch.empty(shape, dtype=torch.int32, device=device)
    info = MaskInfo(B, H, q_len, kv_len, block_q, block_kv, head_masks, q_segment_ids, kv_segment_ids,
                    bmask, dnext, columns=dkv)
    desc, keep = info.mask_desc()
    cinfo = info.info_struct()
    fn = lib.splash_mask_info_build_dkv if dkv else lib.splash_mask_info_build
    st = fn(B, H, q_len, kv_len, block_q, block_kv, ctypes.byref(desc), ctypes.byref(cinfo),
            ctypes.c_void_p(_stream(device)))
    del keep
    _check(st)
    return info


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

_DT = {torch.float32: SPLASH_F32, torch.bfloat16: SPLASH_BF16}


def _strides(t: torch.Tensor, layout: str):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("tensors must be 4-D with a contiguous last (head_dim) axis")
    if layout == "bhsd":
        return _I64x3(t.stride(0), t.stride(1), t.stride(2)), (t.shape[0], t.shape[1], t.shape[2], t.shape[3])
    if layout == "bshd":
        return _I64x3(t.stride(0), t.stride(2), t.stride(1)), (t.shape[0], t.shape[2], t.shape[1], t.shape[3])
    raise ValueError(f"layout must be 'bhsd' or 'bshd', not {layout!r}")


def _forward(pointwise: bool, q, k, v, info: MaskInfo, scale, out, out_dtype, layout):
    lib = load_library()
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    qs, (B, H, Sq, D) = _strides(q, layout)
    ks, (Bk, Hk, Skv, Dk) = _strides(k, layout)
    vs, vshape = _strides(v, layout)
    if (Bk, Dk) != (B, D) or vshape != (B, Hk, Skv, D) or Hk < 1 or H % Hk:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)} ({layout})")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if out_dtype is None:
        out_dtype = q.dtype if out is None else out.dtype
    if out is None:
        shape = (B, H, Sq, D) if layout == "bhsd" else (B, Sq, H, D)
        out = torch.empty(shape, dtype=out_dtype, device=q.device)
    if out.dtype != out_dtype or out.dtype not in _DT:
        raise ValueError("bad output dtype")
    os_, oshape = _strides(out, layout)
    if oshape != (B, H, Sq, D):
        raise ValueError("output shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if (info.B, info.H, info.q_len, info.kv_len) != (B, H, Sq, Skv):
        # the library checks the metadata shape; this catches a different
        # batch/head count that happens to give the same shape
        raise SplashError(SPLASH_ERR_METADATA_MISMATCH,
                          f"metadata built for B={info.B} H={info.H} q_len={info.q_len} kv_len={info.kv_len}")
    desc, keep = info.mask_desc()
    cinfo = info.info_struct()
    tail = (q.data_ptr(), qs, k.data_ptr(), ks, v.data_ptr(), vs, out.data_ptr(), os_,
            float(scale), ctypes.byref(desc), ctypes.byref(cinfo), ctypes.c_void_p(_stream(q.device)))
    if info.dense:
        part = info.partial_struct()
        st = lib.splash_masked_fwd(int(pointwise), _DT[q.dtype], _DT[out_dtype], B, H, Hk, Sq, Skv, D,
                                   *tail[:-1], ctypes.byref(part), tail[-1])
    elif Hk == H:
        fn = lib.splash_pointwise_fwd if pointwise else lib.splash_fwd
        st = fn(_DT[q.dtype], _DT[out_dtype], B, H, Sq, Skv, D, *tail)
    else:
        fn = lib.splash_gqa_pointwise_fwd if pointwise else lib.splash_gqa_fwd
        st = fn(_DT[q.dtype], _DT[out_dtype], B, H, Hk, Sq, Skv, D, *tail)
    del keep
    _check(st)
    return out


def splash_fwd(q, k, v, info: MaskInfo, scale: float | None = None, out=None, out_dtype=None,
               layout: str = "bhsd"):
    """Softmax attention forward under the block-sparse mask of ``info``.

    q [B,H,Sq,D], k/v [B,Hkv,Skv,D] (``layout="bshd"``: [B,S,H,D]); Hkv = H
    is multi-head attention, a divisor of H grouped-query attention (query
    head h reads K/V head h // (H / Hkv)). Default scale 1/sqrt(D). Returns
    ``out`` (allocated if None)."""
    return _forward(False, q, k, v, info, scale, out, out_dtype, layout)


def pointwise_fwd(q, k, v, info: MaskInfo, scale: float | None = None, out=None, out_dtype=None,
                  layout: str = "bhsd"):
    """Pointwise SiLU attention forward: (1/Sq) sum_k silu(scale q.k) v_k;
    k/v may have fewer heads than q, as for ``splash_fwd``."""
    return _forward(True, q, k, v, info, scale, out, out_dtype, layout)


# ---------------------------------------------------------------------------
# pointwise backward
# ---------------------------------------------------------------------------


def _stat_strides(t: torch.Tensor, B: int, H: int, Sq: int):
    """(batch, head) element strides of an fp32 [B, H, Sq] GPU tensor with
    rows contiguous."""
    if t.dtype != torch.float32 or not t.is_cuda or tuple(t.shape) != (B, H, Sq) or (Sq > 1 and t.stride(2) != 1):
        raise ValueError(f"expected a float32 GPU tensor [B, H, Sq] = {(B, H, Sq)} with contiguous rows")
    return _I64x2(t.stride(0), t.stride(1))


def _backward(softmax: bool, q, k, v, d_o, info, info_dkv, scale, out_dtype, layout, out, lse=None, delta=None):
    lib = load_library()
    if q.dtype not in _DT or any(t.dtype != q.dtype for t in (k, v, d_o)):
        raise ValueError("q, k, v, d_o must share dtype float32 or bfloat16")
    if not all(t.is_cuda for t in (q, k, v, d_o)):
        raise ValueError("q, k, v, d_o must be GPU tensors")
    qs, (B, H, Sq, D) = _strides(q, layout)
    ks, (Bk, Hk, Skv, Dk) = _strides(k, layout)
    vs, vshape = _strides(v, layout)
    dos, doshape = _strides(d_o, layout)
    if (Bk, Dk) != (B, D) or vshape != (B, Hk, Skv, D) or doshape != (B, H, Sq, D) or Hk < 1 or H % Hk:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)} "
                         f"d_o {tuple(d_o.shape)} ({layout})")
    if out_dtype is None:
        out_dtype = q.dtype if out is None else out[0].dtype
    if out is None:
        out = (torch.empty_like(q, dtype=out_dtype), torch.empty_like(k, dtype=out_dtype),
               torch.empty_like(v, dtype=out_dtype))
    dq, dk, dv = out
    if any(t.dtype != out_dtype for t in out) or out_dtype not in _DT:
        raise ValueError("bad gradient dtype")
    dqs, dqshape = _strides(dq, layout)
    dks, dkshape = _strides(dk, layout)
    dvs, dvshape = _strides(dv, layout)
    if dqshape != (B, H, Sq, D) or dkshape != (B, Hk, Skv, D) or dvshape != (B, Hk, Skv, D):
        raise ValueError("gradient shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    for m in (info, info_dkv):
        if (m.B, m.H, m.q_len, m.kv_len) != (B, H, Sq, Skv):
            raise SplashError(SPLASH_ERR_METADATA_MISMATCH,
                              f"metadata built for B={m.B} H={m.H} q_len={m.q_len} kv_len={m.kv_len}")
    if info.head_masks != info_dkv.head_masks or info.dense != info_dkv.dense:
        raise ValueError("info and info_dkv were built for different masks")
    if info.columns or not info_dkv.columns:
        raise ValueError("info must come from mask_info_build and info_dkv from mask_info_build_dkv")
    desc, keep = info.mask_desc()
    c1, c2 = info.info_struct(), info_dkv.info_struct()
    head = (_DT[q.dtype], _DT[out_dtype], B, H, Hk, Sq, Skv, D,
            q.data_ptr(), qs, k.data_ptr(), ks, v.data_ptr(), vs, d_o.data_ptr(), dos)
    tail = (dq.data_ptr(), dqs, dk.data_ptr(), dks, dv.data_ptr(), dvs,
            float(scale), ctypes.byref(desc), ctypes.byref(c1), ctypes.byref(c2), ctypes.c_void_p(_stream(q.device)))
    if softmax:
        ss = _stat_strides(lse, B, H, Sq)
        if tuple(_stat_strides(delta, B, H, Sq)) != tuple(ss):
            raise ValueError("lse and delta must share strides")
        stats = (lse.data_ptr(), delta.data_ptr(), ss)
    else:
        stats = (None, None, None)
    if info.dense:
        p1, p2 = info.partial_struct(), info_dkv.partial_struct()
        st = lib.splash_masked_bwd(int(softmax), *head, *stats, *tail[:6], tail[6], tail[7], tail[8],
                                   ctypes.byref(p1), tail[9], ctypes.byref(p2), tail[10])
    elif softmax:
        st = lib.splash_softmax_bwd(*head, *stats, *tail)
    else:
        st = lib.splash_pointwise_bwd(*head, *tail)
    del keep
    _check(st)
    return dq, dk, dv


def pointwise_bwd(q, k, v, d_o, info: MaskInfo, info_dkv: MaskInfo, scale: float | None = None,
                  out_dtype=None, layout: str = "bhsd", out=None):
    """Gradients (dq, dk, dv) of ``pointwise_fwd`` for the output gradient
    ``d_o``: ``info`` from ``mask_info_build`` (dQ pass), ``info_dkv`` from
    ``mask_info_build_dkv`` (dK/dV pass), both for the same mask. k and v may
    have fewer heads than q (a K/V head's gradients sum over its query
    heads). ``out``: an optional (dq, dk, dv) to write into."""
    return _backward(False, q, k, v, d_o, info, info_dkv, scale, out_dtype, layout, out)


# ---------------------------------------------------------------------------
# softmax log-sum-exp and backward
# ---------------------------------------------------------------------------


def splash_fwd_lse(q, k, v, info: MaskInfo, scale: float | None = None, out=None, out_dtype=None,
                   layout: str = "bhsd", lse=None):
    """``splash_fwd`` that also returns the per-row log-sum-exp of the scores
    (fp32 [B, H, Sq]; -inf for rows with no allowed key): (out, lse)."""
    lib = load_library()
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    qs, (B, H, Sq, D) = _strides(q, layout)
    ks, (Bk, Hk, Skv, Dk) = _strides(k, layout)
    vs, vshape = _strides(v, layout)
    if (Bk, Dk) != (B, D) or vshape != (B, Hk, Skv, D) or Hk < 1 or H % Hk:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)} ({layout})")
    if out_dtype is None:
        out_dtype = q.dtype if out is None else out.dtype
    if out is None:
        shape = (B, H, Sq, D) if layout == "bhsd" else (B, Sq, H, D)
        out = torch.empty(shape, dtype=out_dtype, device=q.device)
    os_, oshape = _strides(out, layout)
    if oshape != (B, H, Sq, D) or out.dtype != out_dtype or out_dtype not in _DT:
        raise ValueError("bad output")
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    ls = _stat_strides(lse, B, H, Sq)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if (info.B, info.H, info.q_len, info.kv_len) != (B, H, Sq, Skv):
        raise SplashError(SPLASH_ERR_METADATA_MISMATCH,
                          f"metadata built for B={info.B} H={info.H} q_len={info.q_len} kv_len={info.kv_len}")
    desc, keep = info.mask_desc()
    cinfo = info.info_struct()
    args = (_DT[q.dtype], _DT[out_dtype], B, H, Hk, Sq, Skv, D, q.data_ptr(), qs, k.data_ptr(), ks,
            v.data_ptr(), vs, out.data_ptr(), os_, lse.data_ptr(), ls, float(scale),
            ctypes.byref(desc), ctypes.byref(cinfo))
    if info.dense:
        part = info.partial_struct()
        st = lib.splash_masked_fwd_lse(*args, ctypes.byref(part), ctypes.c_void_p(_stream(q.device)))
    else:
        st = lib.splash_fwd_lse(*args, ctypes.c_void_p(_stream(q.device)))
    del keep
    _check(st)
    return out, lse


def softmax_bwd_preprocess(o, d_o, layout: str = "bhsd", delta=None):
    """delta = rowsum(o * d_o) in fp32 [B, H, Sq] (the softmax backward's
    row term)."""
    lib = load_library()
    if o.dtype not in _DT or d_o.dtype != o.dtype or not (o.is_cuda and d_o.is_cuda):
        raise ValueError("o and d_o must be GPU tensors of one dtype, float32 or bfloat16")
    os_, (B, H, Sq, D) = _strides(o, layout)
    ds_, dshape = _strides(d_o, layout)
    if dshape != (B, H, Sq, D):
        raise ValueError("o and d_o shapes differ")
    if delta is None:
        delta = torch.empty((B, H, Sq), dtype=torch.float32, device=o.device)
    st = lib.splash_softmax_bwd_preprocess(_DT[o.dtype], B, H, Sq, D, o.data_ptr(), os_, d_o.data_ptr(), ds_,
                                           delta.data_ptr(), _stat_strides(delta, B, H, Sq),
                                           ctypes.c_void_p(_stream(o.device)))
    _check(st)
    return delta


def softmax_bwd(q, k, v, d_o, lse, delta, info: MaskInfo, info_dkv: MaskInfo, scale: float | None = None,
                out_dtype=None, layout: str = "bhsd", out=None):
    """Gradients (dq, dk, dv) of ``splash_fwd``, given the forward's ``lse``
    (``splash_fwd_lse``) and ``delta`` (``softmax_bwd_preprocess``); metadata
    as for ``pointwise_bwd``."""
    return _backward(True, q, k, v, d_o, info, info_dkv, scale, out_dtype, layout, out, lse, delta)
