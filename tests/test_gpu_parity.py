"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases (several tiles, ragged tails) are compared element by element;
the full-size workloads are compared on sampled rows that the oracle computes
one by one, in the launch configuration the benchmark times.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import block_sparse_masked_splash_amd as sp
from block_sparse_masked_splash_amd import workloads as wl

from parity_util import check_close, sample_rows, to64

pytestmark = pytest.mark.gpu

CAUSAL, FULL = wl.CAUSAL, wl.FULL


def _seg_np(t):
    return None if t is None else t.numpy()


def _to_dev(c, dev):
    out = {n: (None if c[n] is None else c[n].to(dev)) for n in c}
    return out


def _meta(dev, B, H, Sq, Skv, heads, bq, bkv, g):
    return sp.mask_info_build(B, H, Sq, Skv, heads, bq, bkv, g["q_segment_ids"], g["kv_segment_ids"], device=dev)


# ---------------------------------------------------------------------------
# metadata
# ---------------------------------------------------------------------------

META_CASES = [
    # B, H, Sq, Skv, heads, bq, bkv, segments
    (1, 1, 256, 256, [CAUSAL], 64, 64, None),
    (2, 3, 333, 333, [CAUSAL, wl.local_causal(50), FULL], 64, 64, None),
    (2, 3, 333, 290, [CAUSAL, (0, 20, 70), FULL], 128, 64, None),
    (3, 2, 517, 517, [CAUSAL], 128, 128, "docs"),
    (2, 2, 200, 180, [(1, 30, 30), FULL], 64, 128, "random"),
    (1, 2, 1000, 1000, [CAUSAL, wl.local_causal(100)], 48, 100, None),
    (2, 1, 4100, 4100, [CAUSAL], 64, 64, "docs"),   # more than 64 kv blocks per row
    # segment ids with metadata smaller than the blocks' id ranges (the
    # one-workgroup-per-entry classification), and random ids in ragged blocks
    # of uneven sizes (pair tests on most entries, several 64-query rounds)
    (2, 1, 100, 90, [CAUSAL], 64, 64, "random"),
    (2, 2, 301, 263, [CAUSAL, (0, 40, 10)], 160, 96, "random"),
    (1, 1, 1, 1, [CAUSAL], 64, 64, None),
    (1, 1, 70, 0, [FULL], 64, 64, None),
]


@pytest.mark.parametrize("case", META_CASES, ids=[f"m{n}" for n in range(len(META_CASES))])
def test_mask_info_matches_oracle(gpu_device, case):
    B, H, Sq, Skv, heads, bq, bkv, seg = case
    print(f"mask_info case {case}", flush=True)
    c = wl.random_case(17, B, H, Sq, Skv, 64, "bf16", segments=seg, doc_len=(1, 300))
    g = _to_dev(c, gpu_device)
    info = _meta(gpu_device, B, H, Sq, Skv, heads, bq, bkv, g)
    bm, dn = oracle.mask_info(B, H, Sq, Skv, bq, bkv, heads, _seg_np(c["q_segment_ids"]), _seg_np(c["kv_segment_ids"]))
    np.testing.assert_array_equal(info.block_mask.cpu().numpy(), bm)
    np.testing.assert_array_equal(info.data_next.cpu().numpy(), dn)


@pytest.mark.parametrize("name", ["c1", "c2", "c3h", "c3", "c4", "c5"])
def test_mask_info_full_workloads(gpu_device, name):
    w = wl.WORKLOADS[name]
    print(f"mask_info workload {name}", flush=True)
    rng = np.random.default_rng(w.seed)
    seg = None
    if w.segments:
        g = wl.generate(w)
        seg = g["q_segment_ids"]
        del g
    segd = None if seg is None else seg.to(gpu_device)
    info = sp.mask_info_build(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, segd, segd,
                              device=gpu_device)
    bm = info.block_mask.cpu().numpy()
    dn = info.data_next.cpu().numpy()
    Bm, Hm, nq, nk = bm.shape
    assert (Bm, Hm) == ((w.B if w.segments else 1), len(w.head_masks))
    # every metadata row against the oracle, one row at a time (all rows of
    # every workload with at most 128 of them, which covers the segment-id
    # workload; 40 sampled rows of the 4096 of the mixed-head workload, whose
    # whole arrays are checked against closed forms below)
    if Bm * Hm * nq <= 128:
        rows = {(b, h, i) for b in range(Bm) for h in range(Hm) for i in range(nq)}
    else:
        rows = {(0, 0, 0), (Bm - 1, Hm - 1, nq - 1)}
        while len(rows) < 40:
            rows.add((int(rng.integers(Bm)), int(rng.integers(Hm)), int(rng.integers(nq))))
    segn = None if seg is None else seg.numpy()
    for (b, h, i) in sorted(rows):
        cls, nxt = oracle.mask_info_row(w.S, w.S, w.block_q, w.block_kv, w.head_masks[h], i,
                                        None if segn is None else segn[b], None if segn is None else segn[b])
        np.testing.assert_array_equal(bm[b, h, i], cls, err_msg=f"block_mask row {(b, h, i)}")
        np.testing.assert_array_equal(dn[b, h, i], nxt, err_msg=f"data_next row {(b, h, i)}")
    # whole arrays against the closed forms where there is one
    ii, jj = np.meshgrid(np.arange(nq), np.arange(nk), indexing="ij")
    causal_cls = np.where(jj < ii, 2, np.where(jj == ii, 1, 0))
    for h, head in enumerate(w.head_masks):
        if w.segments:
            # causal AND segments: never more than causal allows
            assert (bm[:, h][:, causal_cls == 0] == 0).all()
            continue
        if head == CAUSAL:
            np.testing.assert_array_equal(bm[0, h], causal_cls)
            np.testing.assert_array_equal(dn[0, h], np.where(jj <= ii, jj, nk))
        else:
            wdw = head[1] // w.block_kv
            want = np.where((jj < ii) & (jj > ii - wdw), 2, np.where((jj == ii) | (jj == ii - wdw), 1, 0))
            np.testing.assert_array_equal(bm[0, h], want)
    if name == "c4":
        assert int((bm[0, 8:] != 0).sum()) == 8 * 2268
        assert int((bm[0, :8] != 0).sum()) == 8 * 32896
    if name == "c3":
        # every non-empty block count agrees with the oracle on the sampled rows; report the total
        print(f"c3 non-empty blocks: {int((bm != 0).sum())} of {Bm * nq * nk}")


# ---------------------------------------------------------------------------
# small forward cases, full comparison
# ---------------------------------------------------------------------------

FWD_CASES = [
    # B, H, Sq, Skv, D, heads, bq, bkv, segments, dtype
    (1, 1, 256, 256, 64, [CAUSAL], 64, 64, None, "f32"),
    (2, 3, 333, 333, 128, [CAUSAL, wl.local_causal(50), FULL], 64, 64, None, "bf16"),
    (2, 3, 333, 333, 128, [CAUSAL, wl.local_causal(50), FULL], 128, 128, None, "bf16"),
    (2, 2, 517, 517, 128, [CAUSAL], 128, 64, "docs", "bf16"),
    (2, 2, 300, 450, 64, [(0, 40, 90), FULL], 64, 128, "random", "bf16"),
    (1, 2, 100, 300, 128, [FULL, CAUSAL], 64, 64, None, "bf16"),
    (2, 2, 190, 190, 128, [CAUSAL, wl.local_causal(33)], 128, 64, "docs", "f32"),
    (1, 3, 130, 257, 64, [FULL, (1, 7, 7), (0, 0, 0)], 64, 128, None, "f32"),
    (2, 2, 600, 600, 128, [CAUSAL, wl.local_causal(100)], 256, 128, "docs", "bf16"),
    (1, 2, 300, 333, 64, [FULL, CAUSAL], 256, 64, None, "bf16"),
    (1, 2, 280, 280, 64, [CAUSAL, (0, 50, 20)], 256, 64, "random", "f32"),
    # fp32 at D = 128 with 256-row q blocks: each q block takes two workgroups
    (2, 2, 300, 270, 128, [CAUSAL, wl.local_causal(90)], 256, 64, "docs", "f32"),
    (1, 2, 517, 517, 128, [FULL, CAUSAL], 256, 128, None, "f32"),
]


@pytest.mark.parametrize("pointwise", [False, True], ids=["softmax", "pointwise"])
@pytest.mark.parametrize("case", FWD_CASES, ids=[f"f{n}" for n in range(len(FWD_CASES))])
def test_forward_small_matches_oracle(gpu_device, case, pointwise):
    B, H, Sq, Skv, D, heads, bq, bkv, seg, dt = case
    print(f"forward case {case} pointwise={pointwise}", flush=True)
    sigma = 0.5 if pointwise else 1.0
    c = wl.random_case(23, B, H, Sq, Skv, D, dt, sigma=sigma, segments=seg, doc_len=(1, 200))
    g = _to_dev(c, gpu_device)
    info = _meta(gpu_device, B, H, Sq, Skv, heads, bq, bkv, g)
    fn = sp.pointwise_fwd if pointwise else sp.splash_fwd
    out = fn(g["q"], g["k"], g["v"], info)
    torch.cuda.synchronize()
    ofn = oracle.pointwise_attention if pointwise else oracle.softmax_attention
    ref = ofn(to64(c["q"]), to64(c["k"]), to64(c["v"]), 1 / math.sqrt(D), heads,
              _seg_np(c["q_segment_ids"]), _seg_np(c["kv_segment_ids"]))
    err = check_close(to64(out), ref, dt, f"{case}")
    print(err)


def test_f32_workload_c1_full(gpu_device):
    w = wl.WORKLOADS["c1"]
    c = wl.generate(w)
    g = _to_dev(c, gpu_device)
    info = _meta(gpu_device, w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, g)
    out = sp.splash_fwd(g["q"], g["k"], g["v"], info, scale=w.scale)
    torch.cuda.synchronize()
    ref = oracle.softmax_attention(to64(c["q"]), to64(c["k"]), to64(c["v"]), w.scale, w.head_masks)
    err = check_close(to64(out), ref, "f32", "c1")
    print("c1", err)


def test_workload_c2_full(gpu_device):
    w = wl.WORKLOADS["c2"]
    c = wl.generate(w)
    g = _to_dev(c, gpu_device)
    info = _meta(gpu_device, w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, g)
    out = sp.splash_fwd(g["q"], g["k"], g["v"], info, scale=w.scale)
    torch.cuda.synchronize()
    ref = oracle.softmax_attention(to64(c["q"]), to64(c["k"]), to64(c["v"]), w.scale, w.head_masks,
                                   row_chunk=1024)
    err = check_close(to64(out), ref, "bf16", "c2")
    print("c2", err)


# ---------------------------------------------------------------------------
# full-size workloads, sampled rows
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["c3h", "c3", "c4", "c5", "g3h", "d3h", "d5"])
def test_full_workload_sampled_rows(gpu_device, name):
    w = wl.WORKLOADS[name]
    print(f"full workload {name}", flush=True)
    c = wl.generate(w)
    g = _to_dev(c, gpu_device)
    dense = None if c["dense"] is None else c["dense"].numpy()
    if dense is not None:
        info = sp.dense_mask_info_build(w.B, w.H, c["dense"], w.head_masks, w.block_q, w.block_kv,
                                        device=gpu_device)
    else:
        info = _meta(gpu_device, w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, g)
    fn = sp.pointwise_fwd if w.pointwise else sp.splash_fwd
    out = fn(g["q"], g["k"], g["v"], info, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1000 + w.seed)
    qs = _seg_np(c["q_segment_ids"])
    # rows at query-block edges (where a block's diagonal kv block starts and
    # ends) and at the sequence ends, besides 400 random rows
    edges = [0, 1, w.block_q - 1, w.block_q, w.block_q + 1, w.S // 2 - 1, w.S // 2, w.S - 2, w.S - 1]
    for i in rng.integers(1, w.S // w.block_q, size=8):
        edges += [int(i) * w.block_q - 1, int(i) * w.block_q]
    rows = sample_rows(rng, w.B, w.H, w.S, 400, sorted(set(edges)))
    if qs is not None:
        # document edges: in every batch row, the first token of each document
        # (it attends to itself alone), the token before it (the end of the
        # previous document), and a random row of each query block that holds
        # a document edge (a block of partial kv blocks)
        more = set()
        for b in range(w.B):
            starts = [t for t in range(1, w.S) if qs[b, t] != qs[b, t - 1]]
            for t in starts:
                h = int(rng.integers(w.H))
                more.add((b, h, t))
                more.add((b, h, t - 1))
                i = t // w.block_q
                more.add((b, int(rng.integers(w.H)), int(rng.integers(i * w.block_q, (i + 1) * w.block_q))))
        assert len(more) >= 20
        rows = sorted(set(rows) | more)
    got, ref = [], []
    cache = {}
    for (b, h, t) in rows:
        hk = oracle.kv_head_of(h, w.H, w.n_kv_heads)
        if (b, hk) not in cache:
            cache.clear()
            cache[(b, hk)] = (to64(c["k"][b, hk]), to64(c["v"][b, hk]))
        k64, v64 = cache[(b, hk)]
        head = w.head_masks[0] if len(w.head_masks) == 1 else w.head_masks[h]
        m = oracle.element_mask(w.S, w.S, head, None if qs is None else qs[b], None if qs is None else qs[b], rows=[t],
                                dense=dense)
        q64 = to64(c["q"][b, h, t:t + 1])
        if w.pointwise:
            r = oracle.pointwise_attention_rows(q64, k64, v64, w.scale, m, w.S)
        else:
            r = oracle.softmax_attention_rows(q64, k64, v64, w.scale, m)
        ref.append(r[0])
        got.append(to64(out[b, h, t]))
    err = check_close(np.stack(got), np.stack(ref), "bf16", name)
    print(name, err)
    if not w.pointwise:
        # causal row 0 and the first token of a document attend only to
        # themselves: the output is exactly that value row
        for (b, h, t) in rows:
            alone = t == 0 or (qs is not None and qs[b, t] != qs[b, t - 1])
            if alone:
                hk = oracle.kv_head_of(h, w.H, w.n_kv_heads)
                assert torch.equal(out[b, h, t].cpu(), c["v"][b, hk, t]), (b, h, t)


# ---------------------------------------------------------------------------
# grouped-query attention (query head h reads K/V head h // (H / kv_heads))
# ---------------------------------------------------------------------------

GQA_CASES = [
    # B, H, kv_heads, Sq, Skv, D, heads, bq, bkv, segments, dtype, layout
    (2, 4, 2, 333, 333, 128, [CAUSAL], 128, 128, None, "bf16", "bhsd"),
    (2, 4, 1, 300, 420, 64, [FULL, CAUSAL, wl.local_causal(40), (0, 30, 60)], 64, 128, "random", "bf16", "bhsd"),
    (1, 8, 2, 517, 517, 128, [CAUSAL], 128, 64, "docs", "bf16", "bshd"),
    (1, 6, 3, 290, 290, 128, [wl.local_causal(70)], 256, 128, None, "bf16", "bhsd"),
    (2, 4, 2, 200, 200, 64, [CAUSAL], 64, 64, "docs", "f32", "bhsd"),
    # units (batch x K/V head) a multiple of 8, three and five per XCD: the
    # XCD work order in groups of 2 and of 4 units, each with a smaller last group
    (3, 8, 8, 200, 200, 64, [CAUSAL], 64, 64, None, "bf16", "bhsd"),
    (1, 80, 40, 130, 130, 128, [CAUSAL, wl.local_causal(30)] * 40, 64, 64, None, "bf16", "bhsd"),
]


@pytest.mark.parametrize("pointwise", [False, True], ids=["softmax", "pointwise"])
@pytest.mark.parametrize("case", GQA_CASES, ids=[f"g{n}" for n in range(len(GQA_CASES))])
def test_gqa_small_matches_oracle(gpu_device, case, pointwise):
    B, H, Hk, Sq, Skv, D, heads, bq, bkv, seg, dt, layout = case
    print(f"gqa case {case} pointwise={pointwise}", flush=True)
    sigma = 0.5 if pointwise else 1.0
    c = wl.random_case(29, B, H, Sq, Skv, D, dt, sigma=sigma, segments=seg, doc_len=(1, 150))
    kv = wl.random_case(31, B, Hk, Sq, Skv, D, dt, sigma=sigma)
    c["k"], c["v"] = kv["k"], kv["v"]
    g = _to_dev(c, gpu_device)
    info = _meta(gpu_device, B, H, Sq, Skv, heads, bq, bkv, g)
    fn = sp.pointwise_fwd if pointwise else sp.splash_fwd
    if layout == "bshd":
        q, k, v = (g[n].transpose(1, 2).contiguous() for n in ("q", "k", "v"))
        out = fn(q, k, v, info, layout="bshd").transpose(1, 2)
    else:
        out = fn(g["q"], g["k"], g["v"], info)
    torch.cuda.synchronize()
    ofn = oracle.pointwise_attention if pointwise else oracle.softmax_attention
    ref = ofn(to64(c["q"]), to64(c["k"]), to64(c["v"]), 1 / math.sqrt(D), heads,
              _seg_np(c["q_segment_ids"]), _seg_np(c["kv_segment_ids"]))
    print(check_close(to64(out), ref, dt, f"gqa {case}"))


# ---------------------------------------------------------------------------
# dense masks (partial blocks carry their own mask bits)
# ---------------------------------------------------------------------------


def _dense(kind, rng, H, Sq, Skv):
    if kind == "tril":
        return np.tri(Sq, Skv, dtype=bool)
    if kind == "random":
        d = rng.random((H, Sq, Skv)) < 0.3
    elif kind == "strided":  # local band plus every 16th key (a global-token pattern)
        q = np.arange(Sq)[:, None]
        k = np.arange(Skv)[None, :]
        d = ((np.abs(q - k) < 24) | (k % 16 == 0))[None].repeat(H, axis=0)
    else:
        raise ValueError(kind)
    n = min(Sq, Skv)
    d[:, np.arange(n), np.arange(n)] = True  # every row keeps a key
    return d


DENSE_CASES = [
    # B, H, kv_heads, Sq, Skv, D, dense, head masks, bq, bkv, dtype
    (2, 2, 2, 333, 333, 128, "random", [FULL], 128, 128, "bf16"),
    (1, 2, 2, 300, 300, 128, "tril", [FULL], 64, 64, "bf16"),
    (1, 4, 2, 517, 400, 128, "strided", [CAUSAL, (0, 100, 100), FULL, CAUSAL], 128, 64, "bf16"),
    (1, 2, 1, 290, 290, 64, "random", [(1, 80, 80)], 256, 128, "bf16"),
    (2, 2, 2, 200, 230, 64, "strided", [FULL], 64, 64, "f32"),
]


@pytest.mark.parametrize("pointwise", [False, True], ids=["softmax", "pointwise"])
@pytest.mark.parametrize("case", DENSE_CASES, ids=[f"n{n}" for n in range(len(DENSE_CASES))])
def test_dense_mask_small_matches_oracle(gpu_device, case, pointwise):
    B, H, Hk, Sq, Skv, D, kind, heads, bq, bkv, dt = case
    print(f"dense case {case} pointwise={pointwise}", flush=True)
    rng = np.random.default_rng(53)
    dense = _dense(kind, rng, H, Sq, Skv)
    sigma = 0.5 if pointwise else 1.0
    c = wl.random_case(47, B, H, Sq, Skv, D, dt, sigma=sigma)
    kv = wl.random_case(59, B, Hk, Sq, Skv, D, dt, sigma=sigma)
    q, k, v = c["q"].to(gpu_device), kv["k"].to(gpu_device), kv["v"].to(gpu_device)
    info = sp.dense_mask_info_build(B, H, torch.from_numpy(dense), heads, bq, bkv, device=gpu_device)
    ref_meta = oracle.mask_info(B, H, Sq, Skv, bq, bkv, heads, dense=dense)
    assert np.array_equal(info.block_mask.cpu().numpy(), ref_meta[0])
    fn = sp.pointwise_fwd if pointwise else sp.splash_fwd
    out = fn(q, k, v, info)
    torch.cuda.synchronize()
    ofn = oracle.pointwise_attention if pointwise else oracle.softmax_attention
    ref = ofn(to64(c["q"]), to64(kv["k"]), to64(kv["v"]), 1 / math.sqrt(D), heads, dense=dense)
    print(check_close(to64(out), ref, dt, f"dense {case}"))


def test_dense_causal_equals_causal_head_mask(gpu_device):
    """A lower-triangular dense mask gives the causal result (bit-identical:
    the same blocks are visited and the same pairs allowed)."""
    B, H, S, D = 1, 2, 520, 128
    c = wl.random_case(61, B, H, S, S, D, "bf16")
    g = _to_dev(c, gpu_device)
    dinfo = sp.dense_mask_info_build(B, H, torch.from_numpy(np.tri(S, S, dtype=bool)), [FULL], 128, 128,
                                     device=gpu_device)
    cinfo = sp.mask_info_build(B, H, S, S, [CAUSAL], 128, 128, device=gpu_device)
    # the full triangle, the ragged last one (8 rows), and 8 full rows left of it
    assert dinfo.mask_blocks.shape[0] == 3
    a = sp.splash_fwd(g["q"], g["k"], g["v"], dinfo)
    b = sp.splash_fwd(g["q"], g["k"], g["v"], cinfo)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dense_mask_large_sampled_rows(gpu_device):
    """Strided dense mask (local band of 24 plus every 16th key) ANDed with
    causal at S=4096, B=1, H=8, D=128, 128x128 blocks; sampled rows."""
    B, H, S, D = 1, 8, 4096, 128
    dense = _dense("strided", None, 1, S, S)[0]
    c = wl.random_case(67, B, H, S, S, D, "bf16")
    g = _to_dev(c, gpu_device)
    info = sp.dense_mask_info_build(B, H, torch.from_numpy(dense), [CAUSAL], 128, 128, device=gpu_device)
    out = sp.splash_fwd(g["q"], g["k"], g["v"], info)
    torch.cuda.synchronize()
    rng = np.random.default_rng(71)
    rows = sample_rows(rng, B, H, S, 40, [127, 128, 2000])
    got, ref = [], []
    for (b, h, t) in rows:
        m = oracle.element_mask(S, S, CAUSAL, rows=[t], dense=dense)
        r = oracle.softmax_attention_rows(to64(c["q"][b, h, t:t + 1]), to64(c["k"][b, h]), to64(c["v"][b, h]),
                                          D ** -0.5, m)
        ref.append(r[0])
        got.append(to64(out[b, h, t]))
    print(check_close(np.stack(got), np.stack(ref), "bf16", "dense large"))


# ---------------------------------------------------------------------------
# layouts, dtypes, edge cases, determinism
# ---------------------------------------------------------------------------


def test_bshd_layout_and_f32_output(gpu_device):
    B, H, S, D = 2, 4, 300, 128
    c = wl.random_case(5, B, H, S, S, D, "bf16")
    heads = [CAUSAL]
    ref = oracle.softmax_attention(to64(c["q"]), to64(c["k"]), to64(c["v"]), D ** -0.5, heads)
    info = sp.mask_info_build(B, H, S, S, heads, 128, 128, device=gpu_device)
    qb, kb, vb = (c[n].transpose(1, 2).contiguous().to(gpu_device) for n in ("q", "k", "v"))  # [B,S,H,D]
    out = sp.splash_fwd(qb, kb, vb, info, layout="bshd")
    out32 = sp.splash_fwd(qb, kb, vb, info, layout="bshd", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out.shape == (B, S, H, D) and out32.dtype == torch.float32
    check_close(to64(out.transpose(1, 2)), ref, "bf16", "bshd")
    err32 = check_close(to64(out32.transpose(1, 2)), ref, "bf16", "bshd-f32out")
    # fp32 output skips the final bf16 rounding: tighter
    assert err32["max_abs"] < 1e-2


def test_empty_and_degenerate_inputs(gpu_device):
    D = 128
    # no batch / no query rows: nothing to do
    for (B, H, S) in [(0, 2, 64), (1, 2, 0)]:
        q = torch.zeros(B, H, S, D, dtype=torch.bfloat16, device=gpu_device)
        info = sp.mask_info_build(B, H, S, S, [CAUSAL], 64, 64, device=gpu_device)
        out = sp.splash_fwd(q, q, q, info)
        assert out.shape == (B, H, S, D)
    # no keys: every row is empty and written as 0
    q = torch.randn(1, 2, 70, D, device=gpu_device).to(torch.bfloat16)
    kv = torch.zeros(1, 2, 0, D, dtype=torch.bfloat16, device=gpu_device)
    info = sp.mask_info_build(1, 2, 70, 0, [FULL], 64, 64, device=gpu_device)
    out = torch.full((1, 2, 70, D), 7.0, dtype=torch.bfloat16, device=gpu_device)
    sp.splash_fwd(q, kv, kv, info, out=out)
    assert (out == 0).all()
    # query segments absent from the kv side: those rows have no allowed key -> 0
    S = 150
    c = wl.random_case(8, 1, 2, S, S, D, "bf16")
    qs = torch.zeros(1, S, dtype=torch.int32)
    qs[0, 100:] = 5
    ks = torch.zeros(1, S, dtype=torch.int32)
    info = sp.mask_info_build(1, 2, S, S, [FULL], 64, 64, qs.to(gpu_device), ks.to(gpu_device), device=gpu_device)
    g = _to_dev(c, gpu_device)
    for fn, ofn in ((sp.splash_fwd, oracle.softmax_attention), (sp.pointwise_fwd, oracle.pointwise_attention)):
        out = fn(g["q"], g["k"], g["v"], info)
        torch.cuda.synchronize()
        assert (out[0, :, 100:] == 0).all()
        ref = ofn(to64(c["q"]), to64(c["k"]), to64(c["v"]), D ** -0.5, [FULL], qs.numpy(), ks.numpy())
        check_close(to64(out), ref, "bf16", fn.__name__)


def test_runs_are_bitwise_deterministic(gpu_device):
    w = wl.WORKLOADS["c2"]
    c = wl.generate(w, B=1, H=4)
    g = _to_dev(c, gpu_device)
    info = _meta(gpu_device, 1, 4, w.S, w.S, w.head_masks, 128, 128, g)
    a = sp.splash_fwd(g["q"], g["k"], g["v"], info)
    b = sp.splash_fwd(g["q"], g["k"], g["v"], info)
    p1 = sp.pointwise_fwd(g["q"], g["k"], g["v"], info)
    p2 = sp.pointwise_fwd(g["q"], g["k"], g["v"], info)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(p1, p2)


def test_tile_size_invariance(gpu_device):
    """Page 3, section 14: kv tiles add up, so the result does not depend on
    the block sizes beyond rounding."""
    B, H, S, D = 1, 4, 512, 128
    c = wl.random_case(9, B, H, S, S, D, "bf16")
    g = _to_dev(c, gpu_device)
    outs = []
    for bq, bkv in ((64, 64), (128, 128), (64, 128), (128, 64), (256, 128), (256, 64)):
        info = sp.mask_info_build(B, H, S, S, [CAUSAL], bq, bkv, device=gpu_device)
        outs.append(to64(sp.splash_fwd(g["q"], g["k"], g["v"], info, out_dtype=torch.float32)))
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 1e-2


def test_large_scores_stay_finite(gpu_device):
    B, H, S, D = 1, 2, 256, 128
    c = wl.random_case(10, B, H, S, S, D, "bf16")
    c["q"] = (c["q"].float() * 30).to(torch.bfloat16)
    g = _to_dev(c, gpu_device)
    info = sp.mask_info_build(B, H, S, S, [CAUSAL], 128, 128, device=gpu_device)
    out = sp.splash_fwd(g["q"], g["k"], g["v"], info)
    torch.cuda.synchronize()
    ref = oracle.softmax_attention(to64(c["q"]), to64(c["k"]), to64(c["v"]), D ** -0.5, [CAUSAL])
    check_close(to64(out), ref, "bf16", "q*30")


@pytest.mark.parametrize("bq,bkv", [(128, 128), (64, 64), (256, 128)])
def test_rising_scores_rescale(gpu_device, bq, bkv):
    """Scores that grow along the key axis by hundreds of units, so the running
    maximum of a row keeps rising block after block and the accumulated
    numerator and denominator must be rescaled many times (page 3, section 15:
    the correction factor applied to l and O when m increases)."""
    B, H, S, D = 1, 2, 640, 128
    c = wl.random_case(11, B, H, S, S, D, "bf16", sigma=0.1)
    ramp = torch.linspace(0.0, 30.0, S).view(1, 1, S, 1)
    c["q"] = (c["q"].float() + 1.0).to(torch.bfloat16)
    c["k"] = (c["k"].float() + ramp).to(torch.bfloat16)
    c["v"] = wl.random_case(12, B, H, S, S, D, "bf16")["v"]
    g = _to_dev(c, gpu_device)
    info = sp.mask_info_build(B, H, S, S, [CAUSAL], bq, bkv, device=gpu_device)
    out = sp.splash_fwd(g["q"], g["k"], g["v"], info)
    torch.cuda.synchronize()
    ref = oracle.softmax_attention(to64(c["q"]), to64(c["k"]), to64(c["v"]), D ** -0.5, [CAUSAL])
    check_close(to64(out), ref, "bf16", f"rising scores {bq}x{bkv}")


def test_metadata_mismatch_raises(gpu_device):
    c = wl.random_case(1, 1, 2, 256, 256, 128, "bf16")
    g = _to_dev(c, gpu_device)
    info = sp.mask_info_build(1, 2, 256, 256, [CAUSAL], 64, 64, device=gpu_device)
    with pytest.raises(sp.SplashError) as e:
        sp.splash_fwd(g["q"][:, :, :128], g["k"], g["v"], info)
    assert e.value.status == 3
