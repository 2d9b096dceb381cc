"""Ragged sequence ends: rows past the end must never reach the result.

Every tensor here is a view into a larger buffer whose rows past the end of
the sequence (in the same head, or the next tokens in [B, S, H, D] layout)
hold NaN. A kernel that reads such a row into a tile multiplies it by a zero
weight at best, and 0 * NaN is NaN, so any read past the end shows up as a
non-finite output. The reads stay inside each buffer, so nothing here can
touch memory outside an allocation. Outputs are also compared with the oracle
on the valid rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import block_sparse_masked_splash_amd as sp
from block_sparse_masked_splash_amd import workloads as wl

from parity_util import check_close, to64

pytestmark = pytest.mark.gpu

CAUSAL, FULL = wl.CAUSAL, wl.FULL
PAD = 96  # rows of NaN after each sequence (more than one 64-row tile)


def _padded(t, layout, dev, pad=PAD):
    """``t`` ([B, H, S, D], CPU) placed at the start of a NaN-filled buffer with
    ``pad`` more rows per sequence; returns the view in ``layout``."""
    B, H, S, D = t.shape
    if layout == "bhsd":
        buf = torch.full((B, H, S + pad, D), float("nan"), dtype=t.dtype, device=dev)
        buf[:, :, :S] = t.to(dev)
        return buf[:, :, :S]
    buf = torch.full((B, S + pad, H, D), float("nan"), dtype=t.dtype, device=dev)
    buf[:, :S] = t.transpose(1, 2).to(dev)
    return buf[:, :S]


def _stat_view(B, H, S, dev):
    """fp32 [B, H, S] view of a NaN-filled [B, H, S + PAD] buffer."""
    return torch.full((B, H, S + PAD), float("nan"), dtype=torch.float32, device=dev)[:, :, :S]


def _bhsd(t, layout):
    return t if layout == "bhsd" else t.transpose(1, 2)


def _seg(c, n):
    return None if c[n] is None else c[n].numpy()


FWD_CASES = [
    # B, H, Hk, Sq, Skv, D, heads, bq, bkv, layout, segments
    (2, 2, 2, 333, 290, 128, [CAUSAL, FULL], 128, 128, "bhsd", None),
    (2, 2, 2, 333, 290, 128, [FULL], 64, 64, "bshd", None),
    (1, 4, 2, 301, 259, 64, [FULL, CAUSAL, wl.local_causal(40), (0, 30, 60)], 128, 128, "bhsd", None),
    (1, 2, 2, 300, 199, 64, [FULL], 256, 64, "bshd", None),
    (2, 2, 1, 333, 290, 128, [FULL], 128, 64, "bhsd", "random"),
    (1, 2, 2, 270, 301, 128, [FULL, CAUSAL], 256, 128, "bshd", "random"),
]


@pytest.mark.parametrize("pointwise", [False, True], ids=["softmax", "pointwise"])
@pytest.mark.parametrize("case", FWD_CASES, ids=[f"t{n}" for n in range(len(FWD_CASES))])
def test_forward_ignores_rows_past_the_end(gpu_device, case, pointwise):
    B, H, Hk, Sq, Skv, D, heads, bq, bkv, layout, seg = case
    print(f"tail forward {case} pointwise={pointwise}", flush=True)
    sigma = 0.5 if pointwise else 1.0
    c = wl.random_case(83, B, H, Sq, Skv, D, "bf16", sigma=sigma, segments=seg)
    kv = wl.random_case(89, B, Hk, Sq, Skv, D, "bf16", sigma=sigma)
    c["k"], c["v"] = kv["k"], kv["v"]
    q, k, v = (_padded(c[n], layout, gpu_device) for n in ("q", "k", "v"))
    qs = None if c["q_segment_ids"] is None else c["q_segment_ids"].to(gpu_device)
    ks = None if c["kv_segment_ids"] is None else c["kv_segment_ids"].to(gpu_device)
    info = sp.mask_info_build(B, H, Sq, Skv, heads, bq, bkv, qs, ks, device=gpu_device)
    fn = sp.pointwise_fwd if pointwise else sp.splash_fwd
    out = _bhsd(fn(q, k, v, info, layout=layout), layout)
    torch.cuda.synchronize()
    got = to64(out)
    assert np.isfinite(got).all(), "a row past the end of a sequence reached the output"
    ofn = oracle.pointwise_attention if pointwise else oracle.softmax_attention
    ref = ofn(to64(c["q"]), to64(c["k"]), to64(c["v"]), 1 / math.sqrt(D), heads, _seg(c, "q_segment_ids"),
              _seg(c, "kv_segment_ids"))
    print(check_close(got, ref, "bf16", f"tail {case}"))


BWD_CASES = [
    # B, H, Hk, Sq, Skv, D, heads, (bq, bkv) row walk, (bq, bkv) column walk, layout
    (2, 2, 2, 333, 290, 64, [FULL, CAUSAL], (128, 128), (128, 128), "bhsd"),
    (1, 2, 2, 333, 290, 128, [FULL], (128, 128), (128, 128), "bshd"),
    (1, 4, 2, 301, 259, 128, [CAUSAL, FULL, wl.local_causal(50), FULL], (64, 64), (64, 64), "bhsd"),
    (1, 2, 2, 300, 270, 64, [FULL], (64, 128), (96, 64), "bshd"),
]


@pytest.mark.parametrize("softmax", [False, True], ids=["pointwise", "softmax"])
@pytest.mark.parametrize("case", BWD_CASES, ids=[f"u{n}" for n in range(len(BWD_CASES))])
def test_backward_ignores_rows_past_the_end(gpu_device, case, softmax):
    B, H, Hk, Sq, Skv, D, heads, (bq, bkv), (cbq, cbkv), layout = case
    print(f"tail backward {case} softmax={softmax}", flush=True)
    sigma = 1.0 if softmax else 0.5
    c = wl.random_case(97, B, H, Sq, Skv, D, "bf16", sigma=sigma)
    kv = wl.random_case(101, B, Hk, Sq, Skv, D, "bf16", sigma=sigma)
    c["k"], c["v"] = kv["k"], kv["v"]
    c["d_o"] = wl.random_case(103, B, H, Sq, Sq, D, "bf16")["q"]
    q, k, v, do = (_padded(c[n], layout, gpu_device) for n in ("q", "k", "v", "d_o"))
    info = sp.mask_info_build(B, H, Sq, Skv, heads, bq, bkv, device=gpu_device)
    info_dkv = sp.mask_info_build_dkv(B, H, Sq, Skv, heads, cbq, cbkv, device=gpu_device)
    q64, k64, v64, do64 = (to64(c[n]) for n in ("q", "k", "v", "d_o"))
    scale = 1 / math.sqrt(D)
    if softmax:
        o = _padded(torch.zeros(B, H, Sq, D, dtype=torch.bfloat16), layout, gpu_device)
        lse = _stat_view(B, H, Sq, gpu_device)
        delta = _stat_view(B, H, Sq, gpu_device)
        sp.splash_fwd_lse(q, k, v, info, layout=layout, out=o, lse=lse)
        sp.softmax_bwd_preprocess(o, do, layout=layout, delta=delta)
        grads = sp.softmax_bwd(q, k, v, do, lse, delta, info, info_dkv, layout=layout)
        ref = oracle.softmax_attention_bwd(q64, k64, v64, do64, scale, heads)
    else:
        grads = sp.pointwise_bwd(q, k, v, do, info, info_dkv, layout=layout)
        ref = oracle.pointwise_attention_bwd(q64, k64, v64, do64, scale, heads)
    torch.cuda.synchronize()
    for name, g, want in zip(("dq", "dk", "dv"), grads, ref):
        got = to64(_bhsd(g, layout))
        assert np.isfinite(got).all(), f"{name}: a row past the end of a sequence reached the gradient"
        print(name, check_close(got, want, "bf16", f"tail {name} {case}"))
