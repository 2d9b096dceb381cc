"""GPU parity of the backwards: the HIP kernels through the C ABI against the
fp64 oracle (``oracle.pointwise_attention_bwd``; ``oracle.softmax_lse`` and
``oracle.softmax_attention_bwd`` for the softmax forward's log-sum-exp and
the softmax backward).

Small cases (several tiles, ragged tails, GQA, segment ids, every supported
block size and dtype) compare dq, dk and dv element by element; the full-size
workload compares sampled dq rows and sampled dk / dv rows, each of which the
oracle forms from one query row or one key column.
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


def _seg(c, n):
    return None if c[n] is None else c[n].numpy()


def _case(seed, B, H, Hk, Sq, Skv, D, dt, seg):
    """q, d_o with H heads, k, v with Hk heads (drawn as separate cases)."""
    c = wl.random_case(seed, B, H, Sq, Skv, D, dt, sigma=0.5, segments=seg, doc_len=(1, 150))
    kv = wl.random_case(seed + 1, B, Hk, Sq, Skv, D, dt, sigma=0.5)
    gr = wl.random_case(seed + 2, B, H, Sq, Sq, D, dt, sigma=1.0)
    c["k"], c["v"], c["d_o"] = kv["k"], kv["v"], gr["q"]
    return c


def _infos(dev, B, H, Sq, Skv, heads, bq, bkv, cbq, cbkv, g):
    qs, ks = g["q_segment_ids"], g["kv_segment_ids"]
    info = sp.mask_info_build(B, H, Sq, Skv, heads, bq, bkv, qs, ks, device=dev)
    info_dkv = sp.mask_info_build_dkv(B, H, Sq, Skv, heads, cbq, cbkv, qs, ks, device=dev)
    return info, info_dkv


DKV_META_CASES = [
    # B, H, Sq, Skv, heads, bq, bkv, segments
    (1, 1, 256, 256, [CAUSAL], 64, 64, None),
    (2, 3, 333, 290, [CAUSAL, (0, 20, 70), FULL], 128, 64, None),
    (3, 2, 517, 517, [CAUSAL, wl.local_causal(40)], 96, 128, "docs"),
    (2, 2, 200, 180, [(1, 30, 30), FULL], 64, 128, "random"),
    (1, 1, 4100, 300, [CAUSAL], 32, 64, None),   # more than 64 q blocks per column
    (2, 1, 90, 100, [CAUSAL], 64, 64, "random"),  # too small to hold the blocks' id ranges
    (2, 2, 263, 301, [CAUSAL, (0, 40, 10)], 96, 160, "random"),
    (1, 1, 4100, 700, [CAUSAL], 32, 64, "docs"),  # more than 64 q blocks per column, with segments
]


@pytest.mark.parametrize("case", DKV_META_CASES, ids=[f"m{n}" for n in range(len(DKV_META_CASES))])
def test_dkv_metadata_matches_oracle(gpu_device, case):
    B, H, Sq, Skv, heads, bq, bkv, seg = case
    print(f"dkv metadata {case}", flush=True)
    c = wl.random_case(3, B, 1, Sq, Skv, 4, "f32", segments=seg, doc_len=(1, 120))
    g = {n: (None if c[n] is None else c[n].to(gpu_device)) for n in ("q_segment_ids", "kv_segment_ids")}
    info = sp.mask_info_build_dkv(B, H, Sq, Skv, heads, bq, bkv, g["q_segment_ids"], g["kv_segment_ids"],
                                  device=gpu_device)
    torch.cuda.synchronize()
    bm, dn = oracle.mask_info_dkv(B, H, Sq, Skv, bq, bkv, heads, _seg(c, "q_segment_ids"), _seg(c, "kv_segment_ids"))
    # stored by columns: [Bm, Hm, nk, nq]
    np.testing.assert_array_equal(info.block_mask.cpu().numpy(), bm.transpose(0, 1, 3, 2))
    np.testing.assert_array_equal(info.data_next.cpu().numpy(), dn.transpose(0, 1, 3, 2))


BWD_CASES = [
    # B, H, Hk, Sq, Skv, D, heads, (bq, bkv) row walk, (bq, bkv) column walk, segments, dtype, out dtype, layout
    (2, 2, 2, 333, 333, 64, [CAUSAL], (128, 128), (128, 128), None, "bf16", "bf16", "bhsd"),
    (2, 2, 2, 333, 333, 128, [CAUSAL, wl.local_causal(50)], (128, 128), (128, 128), None, "bf16", "bf16", "bhsd"),
    (1, 4, 2, 300, 420, 128, [FULL, CAUSAL, wl.local_causal(40), (0, 30, 60)], (64, 128), (64, 64), "random",
     "bf16", "bf16", "bhsd"),
    (1, 4, 1, 517, 517, 64, [CAUSAL], (256, 64), (256, 128), "docs", "bf16", "f32", "bshd"),
    (2, 2, 2, 200, 260, 128, [wl.local_causal(70)], (128, 64), (96, 128), None, "bf16", "bf16", "bhsd"),
    (1, 2, 2, 640, 640, 64, [CAUSAL, FULL], (64, 64), (32, 64), "docs", "bf16", "bf16", "bhsd"),
    (1, 2, 2, 200, 200, 64, [CAUSAL], (64, 64), (64, 64), "docs", "f32", "f32", "bhsd"),
    (1, 2, 1, 130, 190, 128, [CAUSAL, (0, 20, 20)], (128, 128), (64, 64), "random", "f32", "f32", "bhsd"),
    (1, 1, 1, 300, 300, 64, [FULL], (256, 128), (128, 64), None, "f32", "f32", "bhsd"),
    # fp32 at D = 128 with 256-row q blocks: each q block takes two dQ workgroups
    (1, 2, 1, 300, 270, 128, [CAUSAL, wl.local_causal(90)], (256, 64), (64, 128), "docs", "f32", "f32", "bshd"),
    (1, 2, 2, 300, 300, 128, [CAUSAL, FULL], (64, 64), (32, 128), "docs", "bf16", "bf16", "bhsd"),
    # units a multiple of 8 (three or five per XCD): both passes deal them in
    # groups of 2 or 4 with a smaller last group
    (3, 8, 8, 150, 150, 64, [CAUSAL], (64, 64), (64, 64), None, "bf16", "bf16", "bhsd"),
    (1, 80, 40, 130, 130, 128, [CAUSAL], (64, 64), (64, 64), None, "bf16", "bf16", "bhsd"),
    (1, 48, 24, 130, 200, 128, [CAUSAL], (128, 128), (128, 128), None, "bf16", "bf16", "bhsd"),
]


def _run_bwd(dev, case, c):
    B, H, Hk, Sq, Skv, D, heads, (bq, bkv), (cbq, cbkv), seg, dt, odt, layout = case
    g = {n: (None if c[n] is None else c[n].to(dev)) for n in c}
    info, info_dkv = _infos(dev, B, H, Sq, Skv, heads, bq, bkv, cbq, cbkv, g)
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    if layout == "bshd":
        q, k, v, do = (g[n].transpose(1, 2).contiguous() for n in ("q", "k", "v", "d_o"))
        grads = sp.pointwise_bwd(q, k, v, do, info, info_dkv, out_dtype=out_dtype, layout="bshd")
        grads = tuple(t.transpose(1, 2) for t in grads)
    else:
        grads = sp.pointwise_bwd(g["q"], g["k"], g["v"], g["d_o"], info, info_dkv, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"b{n}" for n in range(len(BWD_CASES))])
def test_pointwise_bwd_small_matches_oracle(gpu_device, case):
    B, H, Hk, Sq, Skv, D, heads, _, _, seg, dt, odt, layout = case
    print(f"backward case {case}", flush=True)
    c = _case(41, B, H, Hk, Sq, Skv, D, dt, seg)
    dq, dk, dv = _run_bwd(gpu_device, case, c)
    ref = oracle.pointwise_attention_bwd(to64(c["q"]), to64(c["k"]), to64(c["v"]), to64(c["d_o"]),
                                         1 / math.sqrt(D), heads, _seg(c, "q_segment_ids"),
                                         _seg(c, "kv_segment_ids"))
    tol = "f32" if dt == "f32" else "bf16"
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert got.dtype == (torch.float32 if odt == "f32" else torch.bfloat16)
        print(name, check_close(to64(got), want, tol, f"{name} {case}"))


def test_pointwise_bwd_is_deterministic(gpu_device):
    case = BWD_CASES[2]
    c = _case(43, *case[:6], case[10], case[9])
    a = _run_bwd(gpu_device, case, c)
    b = _run_bwd(gpu_device, case, c)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_pointwise_bwd_block_size_invariance(gpu_device):
    """Other block sizes for either walk visit the same pairs: the gradients
    agree to rounding (bf16) and every masked-out key gets exactly zero."""
    B, H, S, D = 1, 2, 400, 128
    heads = [wl.local_causal(60)]
    c = _case(45, B, H, H, S, S, D, "bf16", None)
    base = (B, H, H, S, S, D, heads, (128, 128), (128, 128), None, "bf16", "f32", "bhsd")
    other = (B, H, H, S, S, D, heads, (64, 64), (256, 64), None, "bf16", "f32", "bhsd")
    a = _run_bwd(gpu_device, base, c)
    b = _run_bwd(gpu_device, other, c)
    for x, y in zip(a, b):
        d = (x - y).abs().max().item()
        assert d <= 2e-2 * x.abs().max().item() + 1e-7, d


def test_pointwise_bwd_empty_sides(gpu_device):
    """No queries: dk = dv = 0 (and nothing read from q or d_o). No keys:
    dq = 0. Rows that no pair reaches are written as zeros."""
    D = 64
    for Sq, Skv in ((0, 100), (100, 0)):
        q = torch.randn(1, 2, Sq, D, device=gpu_device).to(torch.bfloat16)
        k = torch.randn(1, 2, Skv, D, device=gpu_device).to(torch.bfloat16)
        v = torch.randn_like(k)
        do = torch.randn_like(q)
        info = sp.mask_info_build(1, 2, Sq, Skv, [CAUSAL], 64, 64, device=gpu_device)
        info_dkv = sp.mask_info_build_dkv(1, 2, Sq, Skv, [CAUSAL], 64, 64, device=gpu_device)
        out = tuple(torch.full_like(t, 7.0) for t in (q, k, v))
        dq, dk, dv = sp.pointwise_bwd(q, k, v, do, info, info_dkv, out=out)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert (t == 0).all()
    # causal with more keys than queries: keys past the last query get zeros
    S, Skv = 100, 300
    c = _case(47, 1, 1, 1, S, Skv, D, "bf16", None)
    case = (1, 1, 1, S, Skv, D, [CAUSAL], (64, 64), (64, 64), None, "bf16", "bf16", "bhsd")
    c["d_o"] = c["d_o"][:, :, :S]
    dq, dk, dv = _run_bwd(gpu_device, case, c)
    assert (dk[0, 0, S:] == 0).all() and (dv[0, 0, S:] == 0).all()
    assert dk[0, 0, :S].abs().sum() > 0


def test_pointwise_bwd_full_workload_sampled(gpu_device):
    """The backward workload at full size (c5's shape: B=8 H=8 S=4096 D=64,
    causal, 128x128 blocks for both walks): sampled dq rows, and sampled dk /
    dv rows, each from the oracle on one query row or one key column."""
    w = wl.WORKLOADS["b5"]
    print("full backward workload b5", flush=True)
    c = wl.generate(w)
    g = {n: (None if c[n] is None else c[n].to(gpu_device)) for n in ("q", "k", "v", "d_o")}
    info = sp.mask_info_build(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, device=gpu_device)
    info_dkv = sp.mask_info_build_dkv(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, device=gpu_device)
    dq, dk, dv = sp.pointwise_bwd(g["q"], g["k"], g["v"], g["d_o"], info, info_dkv, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1000 + w.seed)
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for _ in range(16):
        b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
        q64, k64, v64, do64 = (to64(c[n][b, h]) for n in ("q", "k", "v", "d_o"))
        rows = sorted({0, w.S - 1, 127, 128, *map(int, rng.integers(0, w.S, 24))})
        m = oracle.element_mask(w.S, w.S, w.head_masks[0], rows=rows)
        a, _, _ = oracle.pointwise_attention_bwd_rows(q64[rows], k64, v64, do64[rows], w.scale, m, w.S)
        got["dq"].append(to64(dq[b, h, rows]))
        ref["dq"].append(a)
        keys = sorted({0, w.S - 1, 127, 128, *map(int, rng.integers(0, w.S, 24))})
        m = oracle.element_mask(w.S, w.S, w.head_masks[0])[:, keys]
        _, bk, bv = oracle.pointwise_attention_bwd_rows(q64, k64[keys], v64[keys], do64, w.scale, m, w.S)
        got["dk"].append(to64(dk[b, h, keys]))
        ref["dk"].append(bk)
        got["dv"].append(to64(dv[b, h, keys]))
        ref["dv"].append(bv)
    for n in ("dq", "dk", "dv"):
        print(n, check_close(np.concatenate(got[n]), np.concatenate(ref[n]), "bf16", f"b5 {n}"))


# ---------------------------------------------------------------------------
# softmax: log-sum-exp, delta, backward
# ---------------------------------------------------------------------------

SM_CASES = [
    # B, H, Hk, Sq, Skv, D, heads, (bq, bkv) row walk, (bq, bkv) column walk, segments, dtype, out dtype, layout
    (2, 2, 2, 333, 333, 128, [CAUSAL, wl.local_causal(50)], (128, 128), (128, 128), None, "bf16", "bf16", "bhsd"),
    (2, 2, 2, 333, 333, 64, [CAUSAL], (128, 128), (128, 128), "docs", "bf16", "bf16", "bhsd"),
    (1, 4, 2, 300, 420, 128, [FULL, CAUSAL, wl.local_causal(40), (0, 30, 60)], (64, 128), (64, 64), "random",
     "bf16", "f32", "bhsd"),
    (1, 4, 1, 517, 517, 64, [CAUSAL], (256, 64), (256, 128), "docs", "bf16", "bf16", "bshd"),
    (1, 2, 2, 200, 200, 64, [CAUSAL], (64, 64), (64, 64), "docs", "f32", "f32", "bhsd"),
    (1, 2, 1, 130, 190, 128, [CAUSAL, (0, 20, 20)], (128, 128), (64, 64), "random", "f32", "f32", "bhsd"),
    (1, 2, 2, 300, 300, 128, [FULL, CAUSAL], (256, 128), (128, 64), "random", "f32", "f32", "bhsd"),
    (1, 2, 2, 250, 250, 128, [CAUSAL, wl.local_causal(60)], (64, 64), (96, 64), "docs", "bf16", "bf16", "bhsd"),
    (1, 48, 24, 130, 200, 128, [CAUSAL], (128, 128), (128, 128), None, "bf16", "bf16", "bhsd"),
]


def _run_softmax(dev, case, c):
    """Forward with log-sum-exp, delta, backward: (out, lse, delta, (dq, dk, dv))."""
    B, H, Hk, Sq, Skv, D, heads, (bq, bkv), (cbq, cbkv), seg, dt, odt, layout = case
    g = {n: (None if c[n] is None else c[n].to(dev)) for n in c}
    info, info_dkv = _infos(dev, B, H, Sq, Skv, heads, bq, bkv, cbq, cbkv, g)
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    if layout == "bshd":
        q, k, v, do = (g[n].transpose(1, 2).contiguous() for n in ("q", "k", "v", "d_o"))
    else:
        q, k, v, do = g["q"], g["k"], g["v"], g["d_o"]
    out, lse = sp.splash_fwd_lse(q, k, v, info, layout=layout)
    delta = sp.softmax_bwd_preprocess(out, do, layout=layout)
    grads = sp.softmax_bwd(q, k, v, do, lse, delta, info, info_dkv, out_dtype=out_dtype, layout=layout)
    torch.cuda.synchronize()
    if layout == "bshd":
        out = out.transpose(1, 2)
        grads = tuple(t.transpose(1, 2) for t in grads)
    return out, lse, delta, grads


@pytest.mark.parametrize("case", SM_CASES, ids=[f"s{n}" for n in range(len(SM_CASES))])
def test_softmax_lse_and_bwd_small_match_oracle(gpu_device, case):
    B, H, Hk, Sq, Skv, D, heads, _, _, seg, dt, odt, layout = case
    print(f"softmax backward case {case}", flush=True)
    c = _case(51, B, H, Hk, Sq, Skv, D, dt, seg)
    out, lse, delta, (dq, dk, dv) = _run_softmax(gpu_device, case, c)
    q64, k64, v64, do64 = (to64(c[n]) for n in ("q", "k", "v", "d_o"))
    qs, ks = _seg(c, "q_segment_ids"), _seg(c, "kv_segment_ids")
    scale = 1 / math.sqrt(D)
    tol = "f32" if dt == "f32" else "bf16"
    # log-sum-exp: rows with no allowed key are -inf on both sides
    want = oracle.softmax_lse(q64, k64, scale, heads, qs, ks)
    got = lse.cpu().double().numpy()
    inf = np.isneginf(want)
    assert (np.isneginf(got) == inf).all()
    d = np.abs(got[~inf] - want[~inf]).max(initial=0.0)
    assert d <= (2e-5 if dt == "f32" else 1e-2), d
    # delta = rowsum(out * d_o) on the library's own output (exact up to fp32 sums)
    dref = (to64(out) * do64).sum(-1)
    assert np.abs(delta.cpu().double().numpy() - dref).max() <= 1e-5 * (1 + np.abs(dref).max())
    ref = oracle.softmax_attention_bwd(q64, k64, v64, do64, scale, heads, qs, ks)
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        print(name, check_close(to64(g), w, tol, f"softmax {name} {case}"))


def test_softmax_bwd_full_workload_sampled(gpu_device):
    """The softmax backward at the headline shape (B=2 H=32 S=8192 D=128,
    causal, 128x128 blocks): sampled dq rows, and dk / dv rows of sampled
    keys, the oracle summing their contributions over all query rows."""
    w = wl.WORKLOADS["s3h"]
    print("full softmax backward workload s3h", flush=True)
    c = wl.generate(w)
    g = {n: c[n].to(gpu_device) for n in ("q", "k", "v", "d_o")}
    info = sp.mask_info_build(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, device=gpu_device)
    info_dkv = sp.mask_info_build_dkv(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, device=gpu_device)
    out, lse = sp.splash_fwd_lse(g["q"], g["k"], g["v"], info, scale=w.scale)
    delta = sp.softmax_bwd_preprocess(out, g["d_o"])
    dq, dk, dv = sp.softmax_bwd(g["q"], g["k"], g["v"], g["d_o"], lse, delta, info, info_dkv, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2000 + w.seed)
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for _ in range(3):
        b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
        q64, k64, v64, do64 = (to64(c[n][b, h]) for n in ("q", "k", "v", "d_o"))
        rows = sorted({0, w.S - 1, 127, 128, *map(int, rng.integers(0, w.S, 40))})
        m = oracle.element_mask(w.S, w.S, w.head_masks[0], rows=rows)
        a, _, _ = oracle.softmax_attention_bwd_rows(q64[rows], k64, v64, do64[rows], w.scale, m)
        got["dq"].append(to64(dq[b, h, rows]))
        ref["dq"].append(a)
        keys = sorted({0, w.S - 1, 127, 128, *map(int, rng.integers(0, w.S, 40))})
        dk_ref = np.zeros((len(keys), w.D))
        dv_ref = np.zeros((len(keys), w.D))
        for r0 in range(0, w.S, 1024):
            rr = np.arange(r0, r0 + 1024)
            m = oracle.element_mask(w.S, w.S, w.head_masks[0], rows=rr)
            _, bk, bv = oracle.softmax_attention_bwd_rows(q64[rr], k64, v64, do64[rr], w.scale, m)
            dk_ref += bk[keys]
            dv_ref += bv[keys]
        got["dk"].append(to64(dk[b, h, keys]))
        ref["dk"].append(dk_ref)
        got["dv"].append(to64(dv[b, h, keys]))
        ref["dv"].append(dv_ref)
    for n in ("dq", "dk", "dv"):
        print(n, check_close(np.concatenate(got[n]), np.concatenate(ref[n]), "bf16", f"s3h {n}"))
