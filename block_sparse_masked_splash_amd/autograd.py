"""Differentiable attention: the forward and backward entry points of the
library as one autograd call.

Sequencing only: the forward is ``splash_fwd_lse`` (softmax) or
``pointwise_fwd``, and the backward is ``softmax_bwd_preprocess`` followed by
``softmax_bwd``, or ``pointwise_bwd``; every step runs in the library's
kernels. The softmax residuals are the forward's output and per-row
log-sum-exp ("JAX 到 VLIW ... 复习笔记", section 15: m + log L), as in the
custom VJP of "hstu_ops.py".
"""

import torch

from . import binding as _b


def _row_contiguous(t: torch.Tensor) -> torch.Tensor:
    # the library needs the head dimension contiguous and rows 16-byte aligned
    if t.stride(-1) == 1 and all(s * t.element_size() % 16 == 0 for s in t.stride()[:-1]) \
            and t.data_ptr() % 16 == 0:
        return t
    return t.contiguous()


class _SplashAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, info, info_dkv, scale, pointwise, layout):
        if pointwise:
            out = _b.pointwise_fwd(q, k, v, info, scale=scale, layout=layout)
            lse = None
        else:
            out, lse = _b.splash_fwd_lse(q, k, v, info, scale=scale, layout=layout)
        ctx.info, ctx.info_dkv, ctx.scale, ctx.pointwise, ctx.layout = info, info_dkv, scale, pointwise, layout
        ctx.save_for_backward(q, k, v, out, *(() if lse is None else (lse,)))
        return out

    @staticmethod
    def backward(ctx, d_out):
        if ctx.info_dkv is None:
            raise RuntimeError("splash_attention: the backward needs info_dkv (mask_info_build_dkv or "
                               "dense_mask_info_build_dkv for the same mask)")
        q, k, v, out, *rest = ctx.saved_tensors
        d_out = _row_contiguous(d_out)
        if ctx.pointwise:
            dq, dk, dv = _b.pointwise_bwd(q, k, v, d_out, ctx.info, ctx.info_dkv, scale=ctx.scale,
                                          layout=ctx.layout)
        else:
            delta = _b.softmax_bwd_preprocess(out, d_out, layout=ctx.layout)
            dq, dk, dv = _b.softmax_bwd(q, k, v, d_out, rest[0], delta, ctx.info, ctx.info_dkv, scale=ctx.scale,
                                        layout=ctx.layout)
        return dq, dk, dv, None, None, None, None, None


def splash_attention(q, k, v, info, info_dkv=None, scale: float | None = None, pointwise: bool = False,
                     layout: str = "bhsd"):
    """Masked attention of q, k, v ([B, H, S, D], or [B, S, H, D] with
    layout="bshd"; k and v may have fewer heads than q) under the mask that
    ``info`` (``mask_info_build`` / ``dense_mask_info_build``) describes:
    softmax, or the pointwise SiLU form with ``pointwise=True``. Differentiable
    in q, k and v when ``info_dkv`` (the dK/dV walk's metadata for the same
    mask) is given. The output has the inputs' dtype."""
    return _SplashAttention.apply(q, k, v, info, info_dkv, scale, pointwise, layout)
