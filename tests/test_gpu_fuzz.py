"""GPU parity over seeded random configurations: shapes, block sizes, head
counts (grouped-query attention included), head masks, segment ids, dtypes
and layouts are drawn at random within the supported ranges, and the
metadata, the forwards and the backwards are compared with the fp64 oracle.

Sizes stay small (sequences of at most 300) so that the oracle evaluates
every case in full.
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

N_FWD = 64
N_BWD = 24


def _head_mask(rng):
    kind = int(rng.integers(4))
    if kind == 0:
        return wl.CAUSAL
    if kind == 1:
        return wl.FULL
    if kind == 2:
        return wl.local_causal(int(rng.integers(1, 120)))
    return (0, int(rng.integers(0, 90)), int(rng.integers(0, 90)))


def _draw(seed, backward):
    rng = np.random.default_rng(1000 + seed)
    # units (batch x K/V heads) are sometimes a multiple of 8, so the XCD work
    # order's unit groups are exercised as well
    B = int(rng.choice([1, 2, 3, 4]))
    Hk = int(rng.choice([1, 2, 4]))
    H = Hk * int(rng.choice([1, 2, 3]))
    Sq = int(rng.integers(1, 300))
    Skv = Sq if rng.random() < 0.5 else int(rng.integers(1, 300))
    D = int(rng.choice([64, 128]))
    bq = int(rng.choice([64, 128, 256]))
    bkv = int(rng.choice([64, 128]))
    nheads = 1 if rng.random() < 0.4 else H
    heads = [_head_mask(rng) for _ in range(nheads)]
    seg = [None, "docs", "random"][int(rng.integers(3))]
    dt = "f32" if (rng.random() < 0.2 and not backward) else "bf16"
    layout = "bshd" if rng.random() < 0.3 else "bhsd"
    return dict(B=B, H=H, Hk=Hk, Sq=Sq, Skv=Skv, D=D, bq=bq, bkv=bkv, heads=heads, seg=seg, dt=dt, layout=layout)


def _inputs(seed, c, sigma):
    g = wl.random_case(seed, c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dt"], sigma=sigma, segments=c["seg"],
                       doc_len=(1, 120))
    kv = wl.random_case(seed + 1, c["B"], c["Hk"], c["Sq"], c["Skv"], c["D"], c["dt"], sigma=sigma)
    g["k"], g["v"] = kv["k"], kv["v"]
    g["d_o"] = wl.random_case(seed + 2, c["B"], c["H"], c["Sq"], c["Sq"], c["D"], c["dt"], sigma=sigma)["q"]
    return g


def _seg(t):
    return None if t is None else t.numpy()


def _dev(g, dev):
    return {n: (None if t is None else t.to(dev)) for n, t in g.items()}


def _to_layout(t, layout):
    return t.transpose(1, 2).contiguous() if layout == "bshd" else t


def _from_layout(t, layout):
    return t.transpose(1, 2) if layout == "bshd" else t


@pytest.mark.parametrize("seed", range(N_FWD))
def test_random_forward_matches_oracle(gpu_device, seed):
    c = _draw(seed, backward=False)
    pointwise = seed % 3 == 2
    print(f"fuzz forward seed {seed}: {c} pointwise={pointwise}", flush=True)
    g = _inputs(7 * seed + 11, c, 0.5 if pointwise else 1.0)
    d = _dev(g, gpu_device)
    info = sp.mask_info_build(c["B"], c["H"], c["Sq"], c["Skv"], c["heads"], c["bq"], c["bkv"],
                              d["q_segment_ids"], d["kv_segment_ids"], device=gpu_device)
    fn = sp.pointwise_fwd if pointwise else sp.splash_fwd
    q, k, v = (_to_layout(d[n], c["layout"]) for n in ("q", "k", "v"))
    out = _from_layout(fn(q, k, v, info, layout=c["layout"]), c["layout"])
    torch.cuda.synchronize()
    bm, dn = oracle.mask_info(c["B"], c["H"], c["Sq"], c["Skv"], c["bq"], c["bkv"], c["heads"],
                              _seg(g["q_segment_ids"]), _seg(g["kv_segment_ids"]))
    assert np.array_equal(info.block_mask.cpu().numpy(), bm)
    assert np.array_equal(info.data_next.cpu().numpy(), dn)
    ofn = oracle.pointwise_attention if pointwise else oracle.softmax_attention
    ref = ofn(to64(g["q"]), to64(g["k"]), to64(g["v"]), 1 / math.sqrt(c["D"]), c["heads"],
              _seg(g["q_segment_ids"]), _seg(g["kv_segment_ids"]))
    print(check_close(to64(out), ref, c["dt"], f"fuzz forward {seed}"))


@pytest.mark.parametrize("seed", range(N_BWD))
def test_random_backward_matches_oracle(gpu_device, seed):
    c = _draw(100 + seed, backward=True)
    c["Skv"] = c["Sq"] if c["seg"] == "docs" else c["Skv"]
    softmax = seed % 2 == 1
    print(f"fuzz backward seed {seed}: {c} softmax={softmax}", flush=True)
    g = _inputs(13 * seed + 5, c, 1.0 if softmax else 0.5)
    d = _dev(g, gpu_device)
    rng = np.random.default_rng(seed)
    cbq, cbkv = int(rng.choice([32, 64, 96, 128])), int(rng.choice([64, 128]))
    info = sp.mask_info_build(c["B"], c["H"], c["Sq"], c["Skv"], c["heads"], c["bq"], c["bkv"],
                              d["q_segment_ids"], d["kv_segment_ids"], device=gpu_device)
    info_dkv = sp.mask_info_build_dkv(c["B"], c["H"], c["Sq"], c["Skv"], c["heads"], cbq, cbkv,
                                      d["q_segment_ids"], d["kv_segment_ids"], device=gpu_device)
    q, k, v, do = (_to_layout(d[n], c["layout"]) for n in ("q", "k", "v", "d_o"))
    L = c["layout"]
    if softmax:
        o, lse = sp.splash_fwd_lse(q, k, v, info, layout=L)
        delta = sp.softmax_bwd_preprocess(o, do, layout=L)
        grads = sp.softmax_bwd(q, k, v, do, lse, delta, info, info_dkv, layout=L)
    else:
        grads = sp.pointwise_bwd(q, k, v, do, info, info_dkv, layout=L)
    torch.cuda.synchronize()
    grads = [_from_layout(t, L) for t in grads]
    ofn = oracle.softmax_attention_bwd if softmax else oracle.pointwise_attention_bwd
    ref = ofn(to64(g["q"]), to64(g["k"]), to64(g["v"]), to64(g["d_o"]), 1 / math.sqrt(c["D"]), c["heads"],
              _seg(g["q_segment_ids"]), _seg(g["kv_segment_ids"]))
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        print(name, check_close_grad(to64(got), want, f"fuzz backward {seed} {name}"))


N_DENSE = 16


@pytest.mark.parametrize("seed", range(N_DENSE))
def test_random_dense_mask_forward_matches_oracle(gpu_device, seed):
    """Arbitrary boolean masks (per head or shared, of random density, with
    runs of allowed keys) ANDed with random head masks, block sizes, head
    counts and dtypes."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.choice([1, 2]))
    Hk = int(rng.choice([1, 2]))
    H = Hk * int(rng.choice([1, 2]))
    Sq, Skv = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    D = int(rng.choice([64, 128]))
    bq, bkv = int(rng.choice([64, 128, 256])), int(rng.choice([64, 128]))
    heads = [_head_mask(rng) for _ in range(1 if rng.random() < 0.5 else H)]
    dt = "f32" if rng.random() < 0.2 else "bf16"
    pointwise = seed % 2 == 1
    # per-head or shared mask: random bits, or runs of allowed keys around a random diagonal
    nh = H if rng.random() < 0.5 else 1
    if rng.random() < 0.5:
        dense = rng.random((nh, Sq, Skv)) < rng.uniform(0.05, 0.9)
    else:
        qi = np.arange(Sq)[:, None]
        ki = np.arange(Skv)[None, :]
        dense = np.stack([np.abs(ki - qi - int(rng.integers(-50, 50))) < int(rng.integers(1, 80)) for _ in range(nh)])
    if nh == 1:
        dense = dense[0]
    print(f"fuzz dense seed {seed}: B={B} H={H} Hk={Hk} Sq={Sq} Skv={Skv} D={D} blocks {bq}x{bkv} heads={heads} "
          f"{dt} pointwise={pointwise} mask heads={nh}", flush=True)
    sigma = 0.5 if pointwise else 1.0
    c = wl.random_case(77 * seed + 3, B, H, Sq, Skv, D, dt, sigma=sigma)
    kv = wl.random_case(77 * seed + 4, B, Hk, Sq, Skv, D, dt, sigma=sigma)
    q, k, v = c["q"].to(gpu_device), kv["k"].to(gpu_device), kv["v"].to(gpu_device)
    info = sp.dense_mask_info_build(B, H, torch.from_numpy(dense), heads, bq, bkv, device=gpu_device)
    bm, dn = oracle.mask_info(B, H, Sq, Skv, bq, bkv, heads, dense=dense)
    assert np.array_equal(info.block_mask.cpu().numpy(), bm)
    assert np.array_equal(info.data_next.cpu().numpy(), dn)
    fn = sp.pointwise_fwd if pointwise else sp.splash_fwd
    out = fn(q, k, v, info)
    torch.cuda.synchronize()
    ofn = oracle.pointwise_attention if pointwise else oracle.softmax_attention
    ref = ofn(to64(c["q"]), to64(kv["k"]), to64(kv["v"]), 1 / math.sqrt(D), heads, dense=dense)
    print(check_close(to64(out), ref, dt, f"fuzz dense {seed}"))


N_ROWS64 = 32


@pytest.mark.parametrize("seed", range(N_ROWS64))
def test_random_rows64_forward_matches_one_block_and_oracle(gpu_device, monkeypatch, seed):
    """The 64-rows-per-wavefront softmax forward (forced on for these small
    cases) over random shapes, band masks, head counts, block sizes, output
    dtypes and layouts: bit-equal to the one-block kernel (outputs and
    log-sum-exp) and within the bf16 bound of the oracle."""
    c = _draw(3000 + seed, backward=False)
    rng = np.random.default_rng(7000 + seed)
    c.update(D=128, seg=None, dt="bf16", bq=int(rng.choice([128, 256])))
    out_dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    print(f"fuzz rows64 seed {seed}: {c} out={out_dtype}", flush=True)
    g = _inputs(17 * seed + 3, c, 1.0)
    d = _dev(g, gpu_device)
    info = sp.mask_info_build(c["B"], c["H"], c["Sq"], c["Skv"], c["heads"], c["bq"], c["bkv"], device=gpu_device)
    q, k, v = (_to_layout(d[n], c["layout"]) for n in ("q", "k", "v"))
    res = {}
    for force in ("1", "0"):
        monkeypatch.setenv("SPLASH_FWD_ROWS64", force)
        out, lse = sp.splash_fwd_lse(q, k, v, info, layout=c["layout"], out_dtype=out_dtype)
        torch.cuda.synchronize()
        res[force] = (_from_layout(out, c["layout"]).cpu(), lse.cpu())
    assert torch.equal(res["1"][0], res["0"][0])
    assert torch.equal(res["1"][1], res["0"][1])
    ref = oracle.softmax_attention(to64(g["q"]), to64(g["k"]), to64(g["v"]), 1 / math.sqrt(c["D"]), c["heads"])
    print(check_close(to64(res["1"][0]), ref, "bf16", f"fuzz rows64 {seed}"))
