"""GPU parity of dense masks in the backward and of dense masks with segment
ids, through the C ABI (splash_masked_fwd, splash_masked_fwd_lse,
splash_masked_bwd) against the fp64 oracle.

The metadata of each walk comes from the host builder
(splash_dense_mask_info_host_ex): rows for the forward and the dQ pass,
columns for the dK/dV pass, each with its own block sizes, with any segment
ids folded into the classes and the partial blocks' bits. The oracle ANDs the
dense array, the head band and segment equality element by element.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import block_sparse_masked_splash_amd as sp
from block_sparse_masked_splash_amd import workloads as wl

from parity_util import check_close, check_close_grad, to64

pytestmark = pytest.mark.gpu

CAUSAL, FULL = wl.CAUSAL, wl.FULL


def _dense(kind, rng, Hd, Sq, Skv):
    if kind == "tril":
        d = np.tri(Sq, Skv, dtype=bool)[None].repeat(Hd, axis=0)
    elif kind == "random":
        d = rng.random((Hd, Sq, Skv)) < 0.4
    elif kind == "strided":  # local band plus every 16th key
        q = np.arange(Sq)[:, None]
        k = np.arange(Skv)[None, :]
        d = ((np.abs(q - k) < 24) | (k % 16 == 0))[None].repeat(Hd, axis=0)
    else:
        raise ValueError(kind)
    n = min(Sq, Skv)
    d[:, np.arange(n), np.arange(n)] = True  # every row keeps a key
    return d


def _ids(rng, kind, B, Sq, Skv):
    if kind is None:
        return None, None
    if kind == "docs":
        qs = wl.draw_documents(rng, B, Sq, 1, 120)
        ks = qs.copy() if Skv == Sq else wl.draw_documents(rng, B, Skv, 1, 120)
    else:
        qs = rng.integers(0, 3, size=(B, Sq)).astype(np.int32)
        ks = rng.integers(0, 3, size=(B, Skv)).astype(np.int32)
    # every query keeps its own key position's id where both exist, so rows with keys stay non-empty
    n = min(Sq, Skv)
    ks[:, :n] = np.where(np.random.default_rng(0).random((B, n)) < 0.5, qs[:, :n], ks[:, :n])
    return qs, ks


FWD_SEG_CASES = [
    # B, H, kv_heads, Sq, Skv, D, dense kind, dense heads, head masks, bq, bkv, segments, dtype
    (2, 2, 2, 333, 333, 128, "tril", 1, [FULL], 128, 128, "docs", "bf16"),
    (2, 4, 2, 300, 300, 64, "random", 4, [CAUSAL], 64, 64, "docs", "bf16"),
    (2, 2, 1, 257, 290, 128, "strided", 1, [(0, 60, 60), FULL], 128, 64, "random", "bf16"),
    (2, 2, 2, 200, 200, 64, "random", 2, [CAUSAL], 64, 128, "docs", "f32"),
]


@pytest.mark.parametrize("pointwise", [False, True], ids=["softmax", "pointwise"])
@pytest.mark.parametrize("case", FWD_SEG_CASES, ids=[f"s{n}" for n in range(len(FWD_SEG_CASES))])
def test_dense_mask_with_segments_forward(gpu_device, case, pointwise):
    B, H, Hk, Sq, Skv, D, kind, Hd, heads, bq, bkv, seg, dt = case
    print(f"dense+segments forward {case} pointwise={pointwise}", flush=True)
    rng = np.random.default_rng(131)
    dense = _dense(kind, rng, Hd, Sq, Skv)
    qs, ks = _ids(rng, seg, B, Sq, Skv)
    sigma = 0.5 if pointwise else 1.0
    c = wl.random_case(137, B, H, Sq, Skv, D, dt, sigma=sigma)
    kv = wl.random_case(139, B, Hk, Sq, Skv, D, dt, sigma=sigma)
    info = sp.dense_mask_info_build(B, H, torch.from_numpy(dense), heads, bq, bkv, device=gpu_device,
                                    q_segment_ids=torch.from_numpy(qs), kv_segment_ids=torch.from_numpy(ks))
    obm, odn = oracle.mask_info(B, H, Sq, Skv, bq, bkv, heads, qs, ks, dense=dense)
    np.testing.assert_array_equal(info.block_mask.cpu().numpy(), obm)
    np.testing.assert_array_equal(info.data_next.cpu().numpy(), odn)
    fn = sp.pointwise_fwd if pointwise else sp.splash_fwd
    out = fn(c["q"].to(gpu_device), kv["k"].to(gpu_device), kv["v"].to(gpu_device), info)
    torch.cuda.synchronize()
    ofn = oracle.pointwise_attention if pointwise else oracle.softmax_attention
    ref = ofn(to64(c["q"]), to64(kv["k"]), to64(kv["v"]), 1 / math.sqrt(D), heads, qs, ks, dense=dense)
    print(check_close(to64(out), ref, dt, f"dense+seg {case}"))


BWD_CASES = [
    # B, H, kv_heads, Sq, Skv, D, dense kind, dense heads, head masks, (bq, bkv) rows, (bq, bkv) columns,
    # segments, dtype, layout
    (2, 2, 2, 333, 333, 64, "random", 2, [CAUSAL], (128, 128), (128, 128), None, "bf16", "bhsd"),
    (1, 4, 2, 300, 270, 64, "strided", 1, [FULL, CAUSAL, (0, 40, 40), FULL], (64, 64), (64, 64), "docs", "bf16",
     "bshd"),
    (2, 2, 2, 333, 333, 128, "random", 2, [FULL], (128, 128), (128, 128), None, "bf16", "bhsd"),
    (1, 4, 1, 290, 310, 128, "strided", 1, [CAUSAL], (64, 128), (96, 64), "random", "bf16", "bhsd"),
    (2, 2, 2, 260, 260, 128, "tril", 1, [FULL], (256, 64), (64, 128), "docs", "bf16", "bshd"),
    (1, 2, 2, 200, 230, 64, "random", 2, [CAUSAL, FULL], (64, 64), (32, 64), "docs", "f32", "bhsd"),
    (1, 2, 1, 150, 150, 128, "strided", 1, [FULL], (128, 128), (64, 128), None, "f32", "bhsd"),
]


@pytest.mark.parametrize("softmax", [False, True], ids=["pointwise", "softmax"])
@pytest.mark.parametrize("case", BWD_CASES, ids=[f"b{n}" for n in range(len(BWD_CASES))])
def test_dense_mask_backward_matches_oracle(gpu_device, case, softmax):
    B, H, Hk, Sq, Skv, D, kind, Hd, heads, (bq, bkv), (cbq, cbkv), seg, dt, layout = case
    print(f"dense backward {case} softmax={softmax}", flush=True)
    rng = np.random.default_rng(149)
    dense = _dense(kind, rng, Hd, Sq, Skv)
    qs, ks = _ids(rng, seg, B, Sq, Skv)
    tq = None if qs is None else torch.from_numpy(qs)
    tk = None if ks is None else torch.from_numpy(ks)
    sigma = 1.0 if softmax else 0.5
    c = wl.random_case(151, B, H, Sq, Skv, D, dt, sigma=sigma)
    kv = wl.random_case(157, B, Hk, Sq, Skv, D, dt, sigma=sigma)
    do = wl.random_case(163, B, H, Sq, Sq, D, dt)["q"]
    dmask = torch.from_numpy(dense)
    info = sp.dense_mask_info_build(B, H, dmask, heads, bq, bkv, device=gpu_device, q_segment_ids=tq,
                                    kv_segment_ids=tk)
    info_dkv = sp.dense_mask_info_build_dkv(B, H, dmask, heads, cbq, cbkv, device=gpu_device, q_segment_ids=tq,
                                            kv_segment_ids=tk)
    # the dK/dV walk's metadata: the same classes by columns, data_next along q blocks
    obm, odn = oracle.mask_info_dkv(B, H, Sq, Skv, cbq, cbkv, heads, qs, ks, dense=dense)
    np.testing.assert_array_equal(info_dkv.block_mask.cpu().numpy(), obm.transpose(0, 1, 3, 2))
    np.testing.assert_array_equal(info_dkv.data_next.cpu().numpy(), odn.transpose(0, 1, 3, 2))
    g = {n: t.to(gpu_device) for n, t in (("q", c["q"]), ("k", kv["k"]), ("v", kv["v"]), ("d_o", do))}
    if layout == "bshd":
        q, k, v, d_o = (g[n].transpose(1, 2).contiguous() for n in ("q", "k", "v", "d_o"))
    else:
        q, k, v, d_o = g["q"], g["k"], g["v"], g["d_o"]
    q64, k64, v64, do64 = to64(c["q"]), to64(kv["k"]), to64(kv["v"]), to64(do)
    scale = 1 / math.sqrt(D)
    tol = "f32" if dt == "f32" else "bf16"
    if softmax:
        out, lse = sp.splash_fwd_lse(q, k, v, info, layout=layout)
        delta = sp.softmax_bwd_preprocess(out, d_o, layout=layout)
        grads = sp.softmax_bwd(q, k, v, d_o, lse, delta, info, info_dkv, layout=layout)
        torch.cuda.synchronize()
        want = oracle.softmax_lse(q64, k64, scale, heads, qs, ks, dense=dense)
        got = lse.cpu().double().numpy()
        inf = np.isneginf(want)
        assert (np.isneginf(got) == inf).all()
        assert np.abs(got[~inf] - want[~inf]).max(initial=0.0) <= (2e-5 if dt == "f32" else 1e-2)
        ref = oracle.softmax_attention_bwd(q64, k64, v64, do64, scale, heads, qs, ks, dense=dense)
    else:
        grads = sp.pointwise_bwd(q, k, v, d_o, info, info_dkv, layout=layout)
        torch.cuda.synchronize()
        ref = oracle.pointwise_attention_bwd(q64, k64, v64, do64, scale, heads, qs, ks, dense=dense)
    # gradients sum up to S bf16-rounded weights each: the relative gradient
    # gates for bf16 (as the randomized backward cases), the fp32 gate for fp32
    for name, gr, w in zip(("dq", "dk", "dv"), grads, ref):
        if layout == "bshd":
            gr = gr.transpose(1, 2)
        if tol == "f32":
            print(name, check_close(to64(gr), w, tol, f"dense {name} {case}"))
        else:
            print(name, check_close_grad(to64(gr), w, f"dense {name} {case}"))


def test_dense_causal_backward_equals_causal_head_mask(gpu_device):
    """The causal pattern as a dense array gives the same gradients as the
    causal head mask: the same blocks are visited with the same pairs."""
    B, H, S, D = 1, 2, 300, 128
    c = wl.random_case(167, B, H, S, S, D, "bf16", sigma=0.5)
    do = wl.random_case(173, B, H, S, S, D, "bf16")["q"].to(gpu_device)
    q, k, v = (c[n].to(gpu_device) for n in ("q", "k", "v"))
    tri = torch.from_numpy(np.tri(S, S, dtype=bool))
    di = sp.dense_mask_info_build(B, H, tri, [FULL], 128, 128, device=gpu_device)
    dk_ = sp.dense_mask_info_build_dkv(B, H, tri, [FULL], 128, 128, device=gpu_device)
    ci = sp.mask_info_build(B, H, S, S, [CAUSAL], 128, 128, device=gpu_device)
    ck = sp.mask_info_build_dkv(B, H, S, S, [CAUSAL], 128, 128, device=gpu_device)
    a = sp.pointwise_bwd(q, k, v, do, di, dk_)
    b = sp.pointwise_bwd(q, k, v, do, ci, ck)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_dense_backward_requires_both_walks(gpu_device):
    """A dense row walk with a head-mask column walk is refused."""
    B, H, S, D = 1, 1, 128, 64
    c = wl.random_case(179, B, H, S, S, D, "bf16")
    q, k, v = (c[n].to(gpu_device) for n in ("q", "k", "v"))
    di = sp.dense_mask_info_build(B, H, torch.from_numpy(np.tri(S, S, dtype=bool)), [FULL], 64, 64,
                                  device=gpu_device)
    ci = sp.mask_info_build_dkv(B, H, S, S, [FULL], 64, 64, device=gpu_device)
    with pytest.raises(ValueError):
        sp.pointwise_bwd(q, k, v, q, di, ci)
