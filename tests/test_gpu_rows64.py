"""GPU parity of the softmax forward's 64-rows-per-wavefront kernel.

At head_dim 128 with a band-only mask and block_q 128 or 256 the library runs
either the one-block kernel or the kernel with 64 query rows per wavefront
(two query blocks per workgroup at block_q 128); by default the second only
for problems with at least 2048 of its workgroups. SPLASH_FWD_ROWS64=1 or 0
picks one of them for every call, so these small cases run both: each is
compared with the oracle, and the two kernels with each other bit for bit
(they form every row with the same arithmetic in the same order).
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

CASES = [
    # B, H, kv_heads, Sq, Skv, heads, bq, bkv, out dtype, layout
    (2, 3, 3, 333, 333, [CAUSAL, wl.local_causal(50), FULL], 128, 128, "bf16", "bhsd"),  # odd q-block count
    (1, 2, 2, 640, 640, [CAUSAL], 128, 64, "bf16", "bhsd"),
    (2, 2, 2, 300, 450, [(0, 40, 90), FULL], 128, 128, "f32", "bhsd"),                 # kv longer than q
    (1, 4, 4, 517, 260, [FULL, CAUSAL, (1, 7, 7), (0, 0, 0)], 128, 64, "bf16", "bhsd"),  # q longer than kv
    (2, 2, 2, 600, 600, [CAUSAL, wl.local_causal(100)], 256, 128, "bf16", "bhsd"),
    (1, 2, 2, 300, 333, [FULL, CAUSAL], 256, 64, "f32", "bhsd"),
    (1, 8, 2, 517, 517, [CAUSAL], 128, 128, "bf16", "bshd"),                           # grouped K/V heads
    (2, 4, 1, 129, 129, [CAUSAL, wl.local_causal(30)] * 2, 128, 128, "bf16", "bhsd"),  # one row past a block
    (1, 1, 1, 1, 1, [CAUSAL], 128, 128, "bf16", "bhsd"),
    (1, 16, 16, 1024, 1024, [CAUSAL], 128, 128, "bf16", "bhsd"),
]


def _run(dev, c, heads, bq, bkv, out_dtype, layout, H, S_q, S_kv):
    B = c["q"].shape[0]
    info = sp.mask_info_build(B, H, S_q, S_kv, heads, bq, bkv, device=dev)
    q, k, v = (c[n].to(dev) for n in ("q", "k", "v"))
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    if layout == "bshd":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
        out, lse = sp.splash_fwd_lse(q, k, v, info, out_dtype=odt, layout="bshd")
        out = out.transpose(1, 2)
    else:
        out, lse = sp.splash_fwd_lse(q, k, v, info, out_dtype=odt)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("case", CASES, ids=[f"r{n}" for n in range(len(CASES))])
def test_rows64_matches_oracle_and_one_block_kernel(gpu_device, monkeypatch, case):
    B, H, Hk, Sq, Skv, heads, bq, bkv, odt, layout = case
    D = 128
    print(f"rows64 case {case}", flush=True)
    c = wl.random_case(41, B, H, Sq, Skv, D, "bf16")
    if Hk != H:
        kv = wl.random_case(43, B, Hk, Sq, Skv, D, "bf16")
        c["k"], c["v"] = kv["k"], kv["v"]
    monkeypatch.setenv("SPLASH_FWD_ROWS64", "1")
    out64, lse64 = _run(gpu_device, c, heads, bq, bkv, odt, layout, H, Sq, Skv)
    monkeypatch.setenv("SPLASH_FWD_ROWS64", "0")
    out1, lse1 = _run(gpu_device, c, heads, bq, bkv, odt, layout, H, Sq, Skv)
    assert torch.equal(out64, out1)
    assert torch.equal(lse64, lse1)
    # (the oracle maps query head h to K/V head h // (H / kv_heads) itself)
    ref = oracle.softmax_attention(to64(c["q"]), to64(c["k"]), to64(c["v"]), 1 / math.sqrt(D), heads)
    check_close(to64(out64), ref, "bf16", f"{case}")
    # log-sum-exp: rows with no allowed key are -inf on both sides; bf16 inputs
    # and bf16-rounded probabilities in L, the bound the other lse tests use
    lse_ref = oracle.softmax_lse(to64(c["q"]), to64(c["k"]), 1 / math.sqrt(D), heads)
    got = lse64.double().numpy()
    inf = np.isneginf(lse_ref)
    assert (np.isneginf(got) == inf).all()
    assert np.abs(got[~inf] - lse_ref[~inf]).max(initial=0.0) <= 1e-2


def test_rows64_rising_scores_rescale(gpu_device, monkeypatch):
    """Scores rising along the keys by hundreds of units: the running maximum
    of every row is raised many times (page 3, section 15), in both row blocks
    of a wavefront."""
    B, H, S, D = 1, 2, 640, 128
    c = wl.random_case(11, B, H, S, S, D, "bf16", sigma=0.1)
    ramp = torch.linspace(0.0, 30.0, S).view(1, 1, S, 1)
    c["q"] = (c["q"].float() + 1.0).to(torch.bfloat16)
    c["k"] = (c["k"].float() + ramp).to(torch.bfloat16)
    c["v"] = wl.random_case(12, B, H, S, S, D, "bf16")["v"]
    monkeypatch.setenv("SPLASH_FWD_ROWS64", "1")
    out, _ = _run(gpu_device, c, [CAUSAL], 128, 128, "bf16", "bhsd", H, S, S)
    ref = oracle.softmax_attention(to64(c["q"]), to64(c["k"]), to64(c["v"]), D ** -0.5, [CAUSAL])
    check_close(to64(out), ref, "bf16", "rows64 rising scores")


def test_rows64_choice_by_size_gives_the_same_result(gpu_device, monkeypatch):
    """Without the override the choice follows the problem size; the result
    is the same either way."""
    B, H, S, D = 2, 32, 2048, 128   # 2 x 32 x 8 = 512 pairs of query blocks: below the threshold
    c = wl.random_case(13, B, H, S, S, D, "bf16")
    monkeypatch.delenv("SPLASH_FWD_ROWS64", raising=False)
    out_default, _ = _run(gpu_device, c, [CAUSAL], 128, 128, "bf16", "bhsd", H, S, S)
    monkeypatch.setenv("SPLASH_FWD_ROWS64", "1")
    out64, _ = _run(gpu_device, c, [CAUSAL], 128, 128, "bf16", "bhsd", H, S, S)
    assert torch.equal(out_default, out64)


def _nan_padded(t, layout, dev, pad=96):
    """``t`` ([B, H, S, D], CPU) at the start of a NaN-filled buffer with
    ``pad`` more rows per sequence, as a view in ``layout``."""
    B, H, S, D = t.shape
    if layout == "bhsd":
        buf = torch.full((B, H, S + pad, D), float("nan"), dtype=t.dtype, device=dev)
        buf[:, :, :S] = t.to(dev)
        return buf[:, :, :S]
    buf = torch.full((B, S + pad, H, D), float("nan"), dtype=t.dtype, device=dev)
    buf[:, :S] = t.transpose(1, 2).to(dev)
    return buf[:, :S]


@pytest.mark.parametrize("case", [
    # B, H, kv_heads, Sq, Skv, heads, bq, bkv, layout
    (2, 2, 2, 333, 290, [CAUSAL, FULL], 128, 128, "bhsd"),
    (1, 4, 2, 301, 259, [FULL, CAUSAL, wl.local_causal(40), (0, 30, 60)], 256, 128, "bshd"),
    (1, 2, 1, 270, 301, [FULL, CAUSAL], 128, 64, "bshd"),
], ids=["n0", "n1", "n2"])
def test_rows64_ignores_rows_past_the_end(gpu_device, monkeypatch, case):
    """Ragged ends with NaN in every row past each sequence end (views into
    larger buffers): a tile row read past the end would reach the output as
    NaN through a zero weight."""
    B, H, Hk, Sq, Skv, heads, bq, bkv, layout = case
    D = 128
    print(f"rows64 tail case {case}", flush=True)
    c = wl.random_case(47, B, H, Sq, Skv, D, "bf16")
    kv = wl.random_case(53, B, Hk, Sq, Skv, D, "bf16")
    q, k, v = _nan_padded(c["q"], layout, gpu_device), _nan_padded(kv["k"], layout, gpu_device), \
        _nan_padded(kv["v"], layout, gpu_device)
    info = sp.mask_info_build(B, H, Sq, Skv, heads, bq, bkv, device=gpu_device)
    monkeypatch.setenv("SPLASH_FWD_ROWS64", "1")
    out, lse = sp.splash_fwd_lse(q, k, v, info, layout=layout)
    torch.cuda.synchronize()
    out = out if layout == "bhsd" else out.transpose(1, 2)
    assert torch.isfinite(out.float()).all()
    ref = oracle.softmax_attention(to64(c["q"]), to64(kv["k"]), to64(kv["v"]), 1 / math.sqrt(D), heads)
    check_close(to64(out.cpu()), ref, "bf16", f"{case}")


def test_rows64_no_keys_and_no_queries(gpu_device, monkeypatch):
    """No keys: every row is empty, written as 0 with log-sum-exp -inf; no
    query rows: nothing is launched."""
    D = 128
    monkeypatch.setenv("SPLASH_FWD_ROWS64", "1")
    q = torch.randn(1, 2, 300, D, device=gpu_device).to(torch.bfloat16)
    kv = torch.zeros(1, 2, 0, D, dtype=torch.bfloat16, device=gpu_device)
    info = sp.mask_info_build(1, 2, 300, 0, [FULL, CAUSAL], 128, 128, device=gpu_device)
    out = torch.full((1, 2, 300, D), 7.0, dtype=torch.bfloat16, device=gpu_device)
    _, lse = sp.splash_fwd_lse(q, kv, kv, info, out=out)
    torch.cuda.synchronize()
    assert (out == 0).all()
    assert torch.isneginf(lse).all()
    q0 = torch.zeros(1, 2, 0, D, dtype=torch.bfloat16, device=gpu_device)
    info0 = sp.mask_info_build(1, 2, 0, 0, [CAUSAL], 128, 128, device=gpu_device)
    assert sp.splash_fwd(q0, q0, q0, info0).shape == (1, 2, 0, D)
