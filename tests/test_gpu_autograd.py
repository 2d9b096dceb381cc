"""GPU tests of ``splash_attention``, the differentiable wrapper: its
gradients through torch autograd equal the direct backward calls bit for bit
and match the oracle's gradients (softmax and pointwise, grouped K/V heads,
both layouts); a backward without the dK/dV metadata raises."""

import math

import pytest
import torch

import oracle
import block_sparse_masked_splash_amd as sp
from block_sparse_masked_splash_amd import workloads as wl

from parity_util import check_close, check_close_grad, to64

pytestmark = pytest.mark.gpu

CAUSAL, FULL = wl.CAUSAL, wl.FULL

CASES = [
    # B, H, kv_heads, S, D, heads, (bq, bkv), (bq, bkv) of the dK/dV walk, pointwise, layout, segments
    (2, 4, 2, 300, 128, [CAUSAL, wl.local_causal(60), FULL, CAUSAL], (128, 128), (128, 128), False, "bhsd", None),
    (1, 2, 2, 257, 64, [CAUSAL], (64, 64), (64, 128), True, "bshd", "docs"),
    (1, 3, 1, 200, 128, [FULL, CAUSAL, (0, 20, 20)], (128, 64), (64, 64), False, "bshd", "random"),
]


def _lay(t, layout):
    return t.transpose(1, 2).contiguous() if layout == "bshd" else t.contiguous()


def _unlay(t, layout):
    return t.transpose(1, 2) if layout == "bshd" else t


@pytest.mark.parametrize("case", CASES, ids=[f"a{n}" for n in range(len(CASES))])
def test_autograd_matches_direct_calls_and_oracle(gpu_device, case):
    B, H, Hk, S, D, heads, (bq, bkv), (cbq, cbkv), pointwise, layout, seg = case
    print(f"autograd case {case}", flush=True)
    sigma = 0.5 if pointwise else 1.0
    c = wl.random_case(61, B, H, S, S, D, "bf16", sigma=sigma, segments=seg, doc_len=(1, 100))
    kv = wl.random_case(67, B, Hk, S, S, D, "bf16", sigma=sigma)
    c["k"], c["v"] = kv["k"], kv["v"]
    g = wl.random_case(71, B, H, S, S, D, "bf16")["q"]  # output gradient, bf16
    qs = None if c["q_segment_ids"] is None else c["q_segment_ids"].to(gpu_device)
    ks = None if c["kv_segment_ids"] is None else c["kv_segment_ids"].to(gpu_device)
    info = sp.mask_info_build(B, H, S, S, heads, bq, bkv, qs, ks, device=gpu_device)
    info_dkv = sp.mask_info_build_dkv(B, H, S, S, heads, cbq, cbkv, qs, ks, device=gpu_device)
    q, k, v = (_lay(c[n], layout).to(gpu_device).requires_grad_(True) for n in ("q", "k", "v"))
    d_o = _lay(g, layout).to(gpu_device)

    out = sp.splash_attention(q, k, v, info, info_dkv, pointwise=pointwise, layout=layout)
    (out.float() * d_o.float()).sum().backward()
    torch.cuda.synchronize()

    # the same calls made directly
    qd, kd, vd = (t.detach() for t in (q, k, v))
    if pointwise:
        out_d = sp.pointwise_fwd(qd, kd, vd, info, layout=layout)
        grads = sp.pointwise_bwd(qd, kd, vd, d_o, info, info_dkv, layout=layout)
    else:
        out_d, lse = sp.splash_fwd_lse(qd, kd, vd, info, layout=layout)
        delta = sp.softmax_bwd_preprocess(out_d, d_o, layout=layout)
        grads = sp.softmax_bwd(qd, kd, vd, d_o, lse, delta, info, info_dkv, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), out_d)
    for got, want in zip((q.grad, k.grad, v.grad), grads):
        assert got.dtype == torch.bfloat16
        assert torch.equal(got, want)

    # and the oracle's gradients of the definition
    qn, kn = c["q_segment_ids"], c["kv_segment_ids"]
    qn = None if qn is None else qn.numpy()
    kn = None if kn is None else kn.numpy()
    fwd = oracle.pointwise_attention if pointwise else oracle.softmax_attention
    bwd = oracle.pointwise_attention_bwd if pointwise else oracle.softmax_attention_bwd
    args = (to64(c["q"]), to64(c["k"]), to64(c["v"]))
    check_close(to64(_unlay(out.detach(), layout).cpu()), fwd(*args, 1 / math.sqrt(D), heads, qn, kn), "bf16",
                f"{case} out")
    refs = bwd(*args, to64(g), 1 / math.sqrt(D), heads, qn, kn)
    for name, got, want in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), refs):
        print(name, check_close_grad(to64(_unlay(got, layout).cpu()), want, f"{case} {name}"))


def test_autograd_without_dkv_metadata_raises(gpu_device):
    c = wl.random_case(73, 1, 2, 100, 100, 64, "bf16")
    info = sp.mask_info_build(1, 2, 100, 100, [CAUSAL], 64, 64, device=gpu_device)
    q, k, v = (c[n].to(gpu_device).requires_grad_(True) for n in ("q", "k", "v"))
    out = sp.splash_attention(q, k, v, info)
    with pytest.raises(RuntimeError, match="info_dkv"):
        out.float().sum().backward()
