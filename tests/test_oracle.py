"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Nothing here re-types the oracle's own formulas: every check is a printed
value, a closed form, a special case reducing to a library routine, an
independent brute force, or an invariant. Runs on the CPU.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_masked_splash_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CAUSAL, FULL = (1, -1, -1), (0, -1, -1)


def _f64(t):
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# metadata
# ---------------------------------------------------------------------------


def test_page3_worked_data_next_example():
    """Page 3, section 21: valid = 1 0 0 1 0 1 -> data_next[1] = data_next[2] = 3."""
    with open(os.path.join(GOLDEN, "page3_sec21_data_next.json")) as f:
        g = json.load(f)
    dn = oracle.next_nonempty(g["valid"])
    for j, want in g["printed_data_next"].items():
        assert dn[int(j)] == want
    # a valid block points at itself; past the last valid block there is nothing
    for j, v in enumerate(g["valid"]):
        if v:
            assert dn[j] == j
    assert list(oracle.next_nonempty([0, 0, 0])) == [3, 3, 3]
    assert list(oracle.next_nonempty([])) == []


@pytest.mark.parametrize("S,b", [(256, 64), (1024, 128), (512, 64)])
def test_causal_metadata_closed_form(S, b):
    bm, dn = oracle.mask_info(1, 1, S, S, b, b, [CAUSAL])
    n = S // b
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    want = np.where(j < i, 2, np.where(j == i, 1, 0))
    np.testing.assert_array_equal(bm[0, 0], want)
    np.testing.assert_array_equal(dn[0, 0], np.where(j <= i, j, n))
    assert np.count_nonzero(bm) == n * (n + 1) // 2


def test_workload_block_counts_and_flops():
    """Non-empty block counts n(n+1)/2 of the causal workloads and the FLOP
    count of the S=8192 workload (4*128*128*128 per block, 64 (b, h))."""
    for name, want in [("c1", 10), ("c2", 136), ("c5", 528)]:
        w = wl.WORKLOADS[name]
        bm, _ = oracle.mask_info(1, 1, w.S, w.S, w.block_q, w.block_kv, w.head_masks)
        assert np.count_nonzero(bm) == want
    n = 64
    bm = np.tril(np.ones((n, n), dtype=np.int8))[None, None]
    assert oracle.block_flops(bm, 2, 32, 128, 128, 128) == 133120 * 4 * 128 ** 3
    assert abs(oracle.block_flops(bm, 2, 32, 128, 128, 128) - 1.1167e12) < 1e8


def test_local_window_metadata_closed_form():
    """Causal AND window 1024 at 128x128 blocks: rows i >= 8 have partial
    blocks {i-8, i} and full blocks i-7..i-1; rows i < 8 have i+1 blocks. At
    nq = 256 that is 36 + 9*248 = 2268 non-empty blocks per head."""
    S, b, w = 4096, 128, 1024
    bm, dn = oracle.mask_info(1, 1, S, S, b, b, [wl.local_causal(w)])
    n = S // b
    for i in range(n):
        row = bm[0, 0, i]
        if i >= 8:
            assert row[i - 8] == 1 and row[i] == 1
            assert (row[i - 7:i] == 2).all()
            assert (row[:i - 8] == 0).all() and (row[i + 1:] == 0).all()
            assert dn[0, 0, i, 0] == i - 8
        else:
            assert row[i] == 1 and (row[:i] == 2).all() and (row[i + 1:] == 0).all()
    assert np.count_nonzero(bm) == 36 + 9 * (n - 8)
    assert 36 + 9 * (256 - 8) == 2268


def test_element_counts_closed_form():
    """Allowed pairs: causal S(S+1)/2; causal window w: sum_q min(q, w) + 1.
    A window off by one (k > q - w, or k >= q - w + 1) fails the second."""
    S, w = 300, 37
    assert oracle.element_mask(S, S, CAUSAL).sum() == S * (S + 1) // 2
    assert oracle.element_mask(S, S, wl.local_causal(w)).sum() == sum(min(q, w) + 1 for q in range(S))
    assert oracle.element_mask(S, S, FULL).sum() == S * S
    # symmetric window without causal: |q - k| <= w
    m = oracle.element_mask(S, S, (0, w, w))
    assert m.sum() == sum(min(q, w) + 1 + min(S - 1 - q, w) for q in range(S))


def test_element_flops_closed_forms(monkeypatch):
    """The element-exact FLOP count, 4*D per allowed (q, k) pair over every
    (batch, head), against closed forms: causal S(S+1)/2 pairs per head (at
    the S=8192 workload that is 1.0997e12 FLOPs), causal window w sum_q
    min(q, w) + 1, full Sq*Skv, causal with Sq != Skv sum_q min(q + 1, Skv),
    causal AND same document sum over documents L(L+1)/2, the causal pattern
    as a dense array, and per-head masks summed head by head."""
    import oracle.splash_oracle as so

    D = 64
    S, w = 300, 37
    tri = S * (S + 1) // 2
    win = sum(min(q, w) + 1 for q in range(S))
    assert oracle.element_flops(2, 3, S, S, D, [CAUSAL]) == 4 * D * 2 * 3 * tri
    assert oracle.element_flops(1, 3, S, S, D, [CAUSAL, wl.local_causal(w), FULL]) == 4 * D * (tri + win + S * S)
    assert oracle.element_flops(1, 1, 200, 300, D, [CAUSAL]) == 4 * D * sum(min(q + 1, 300) for q in range(200))
    assert oracle.element_flops(1, 1, 300, 200, D, [CAUSAL]) == 4 * D * sum(min(q + 1, 200) for q in range(300))
    assert oracle.element_flops(1, 2, 120, 70, D, [FULL]) == 4 * D * 2 * 120 * 70
    # packed documents: causal AND same document gives each document its own triangle
    lens = [[50, 120, 30, 100], [300]]
    ids = np.array([np.repeat(np.arange(len(L)), L) for L in lens], dtype=np.int32)
    want = sum(L * (L + 1) // 2 for row in lens for L in row)
    assert oracle.element_flops(2, 2, S, S, D, [CAUSAL], ids, ids) == 4 * D * 2 * want
    assert oracle.element_flops(2, 1, S, S, D, [FULL], ids, ids) == 4 * D * sum(L * L for row in lens for L in row)
    # the causal pattern written out as a dense array (shared, and per head)
    assert oracle.element_flops(1, 2, S, S, D, [FULL], dense=np.tri(S, S, dtype=bool)) == 4 * D * 2 * tri
    dh = np.stack([np.tri(S, S, dtype=bool), np.ones((S, S), dtype=bool)])
    assert oracle.element_flops(1, 2, S, S, D, [FULL], dense=dh) == 4 * D * (tri + S * S)
    # full-size workloads: causal B=2 H=32 S=8192 D=128, and the mixed-head S=32768 workload
    n = 8192
    f = oracle.element_flops(2, 32, n, n, 128, [CAUSAL])
    assert f == 4 * 128 * 64 * n * (n + 1) // 2
    assert abs(f - 1.0997e12) < 1e8
    w4 = wl.WORKLOADS["c4"]
    n, w = 32768, 1024
    local = w * (w + 1) // 2 + (n - w) * (w + 1)
    assert oracle.element_flops(1, 16, n, n, 128, w4.head_masks) == 4 * 128 * 8 * (n * (n + 1) // 2 + local)
    # a count that drops the diagonal (S(S-1)/2 pairs) fails the causal pin
    real = so.element_mask

    def no_diagonal(q_len, kv_len, head, *a, **k):
        m = real(q_len, kv_len, head, *a, **k)
        return m & ~np.eye(q_len, kv_len, dtype=bool)

    monkeypatch.setattr(so, "element_mask", no_diagonal)
    assert so.element_flops(1, 1, S, S, D, [CAUSAL]) != 4 * D * tri


def test_head_broadcast_and_per_head_metadata():
    heads = [CAUSAL, wl.local_causal(64), FULL]
    bm, dn = oracle.mask_info(1, 3, 512, 512, 64, 64, heads)
    for h, hd in enumerate(heads):
        one, one_dn = oracle.mask_info(1, 1, 512, 512, 64, 64, [hd])
        np.testing.assert_array_equal(bm[:, h], one[:, 0])
        np.testing.assert_array_equal(dn[:, h], one_dn[:, 0])
    assert (bm[0, 2] == 2).all()  # FULL: every block full


def test_aligned_documents_metadata():
    """Documents exactly one block long under causal AND segment: only the
    diagonal blocks run and each is partial; two blocks long: the block below
    the diagonal inside a document is full."""
    b, n = 64, 6
    S = b * n
    ids = np.repeat(np.arange(n, dtype=np.int32), b)[None]
    bm, dn = oracle.mask_info(1, 1, S, S, b, b, [CAUSAL], ids, ids)
    np.testing.assert_array_equal(bm[0, 0], np.eye(n, dtype=np.int8))
    np.testing.assert_array_equal(dn[0, 0], np.where(np.arange(n)[None] <= np.arange(n)[:, None],
                                                     np.arange(n)[:, None], n))
    ids2 = np.repeat(np.arange(n // 2, dtype=np.int32), 2 * b)[None]
    bm2, _ = oracle.mask_info(1, 1, S, S, b, b, [CAUSAL], ids2, ids2)
    want = np.eye(n, dtype=np.int8)
    for d in range(n // 2):
        want[2 * d + 1, 2 * d] = 2
    np.testing.assert_array_equal(bm2[0, 0], want)


def test_ragged_metadata():
    """Blocks that extend past the sequence end are never full."""
    bm, dn = oracle.mask_info(1, 1, 200, 200, 64, 64, [FULL])
    assert bm.shape == (1, 1, 4, 4)
    assert (bm[0, 0, :3, :3] == 2).all()
    assert (bm[0, 0, 3, :] == 1).all() and (bm[0, 0, :, 3] == 1).all()
    bm, dn = oracle.mask_info(1, 1, 0, 0, 64, 64, [FULL])
    assert bm.shape == (1, 1, 0, 0)
    bm, dn = oracle.mask_info(1, 1, 100, 0, 64, 64, [FULL])
    assert bm.shape == (1, 1, 2, 0)


def test_metadata_brute_force_small():
    """Block classes by scalar loops over every (q, k) pair, random windows,
    segments and ragged lengths."""
    rng = np.random.default_rng(7)
    for trial in range(6):
        Sq, Skv = int(rng.integers(1, 70)), int(rng.integers(1, 70))
        bq, bkv = int(rng.choice([4, 8, 16])), int(rng.choice([4, 8, 16]))
        head = (int(rng.integers(0, 2)), int(rng.integers(-1, 12)), int(rng.integers(-1, 12)))
        qs = rng.integers(0, 3, size=(1, Sq)).astype(np.int32)
        ks = rng.integers(0, 3, size=(1, Skv)).astype(np.int32)
        bm, dn = oracle.mask_info(1, 1, Sq, Skv, bq, bkv, [head], qs, ks)
        nq, nk = -(-Sq // bq), -(-Skv // bkv)
        for i in range(nq):
            for j in range(nk):
                c = 0
                for q in range(i * bq, (i + 1) * bq):
                    for k in range(j * bkv, (j + 1) * bkv):
                        if q >= Sq or k >= Skv:
                            continue
                        ok = (not head[0] or k <= q) and (head[1] < 0 or k >= q - head[1]) \
                            and (head[2] < 0 or k <= q + head[2]) and qs[0, q] == ks[0, k]
                        c += bool(ok)
                want = 0 if c == 0 else (2 if c == bq * bkv else 1)
                assert bm[0, 0, i, j] == want
            for j in range(nk):
                nxt = next((jj for jj in range(j, nk) if bm[0, 0, i, jj]), nk)
                assert dn[0, 0, i, j] == nxt


# ---------------------------------------------------------------------------
# dense masks
# ---------------------------------------------------------------------------


def test_dense_lower_triangle_is_the_causal_mask():
    """A dense mask holding the lower triangle reduces to the causal head mask:
    same element mask, same metadata."""
    Sq, Skv, bq, bkv = 200, 230, 32, 64
    tril = np.tri(Sq, Skv, dtype=bool)
    np.testing.assert_array_equal(oracle.element_mask(Sq, Skv, FULL, dense=tril),
                                  oracle.element_mask(Sq, Skv, CAUSAL))
    a = oracle.mask_info(1, 1, Sq, Skv, bq, bkv, [FULL], dense=tril)
    c = oracle.mask_info(1, 1, Sq, Skv, bq, bkv, [CAUSAL])
    np.testing.assert_array_equal(a[0], c[0])
    np.testing.assert_array_equal(a[1], c[1])


def test_dense_metadata_brute_force_small():
    """Block classes of dense masks ANDed with head bands, by scalar loops."""
    rng = np.random.default_rng(19)
    for trial in range(6):
        Sq, Skv = int(rng.integers(1, 60)), int(rng.integers(1, 60))
        bq, bkv = int(rng.choice([4, 8, 16])), int(rng.choice([4, 8, 16]))
        head = (int(rng.integers(0, 2)), int(rng.integers(-1, 12)), int(rng.integers(-1, 12)))
        dense = rng.random((Sq, Skv)) < rng.choice([0.05, 0.5, 0.95])
        bm, dn = oracle.mask_info(1, 1, Sq, Skv, bq, bkv, [head], dense=dense)
        nq, nk = -(-Sq // bq), -(-Skv // bkv)
        for i in range(nq):
            for j in range(nk):
                c = 0
                for q in range(i * bq, min(Sq, (i + 1) * bq)):
                    for k in range(j * bkv, min(Skv, (j + 1) * bkv)):
                        ok = (not head[0] or k <= q) and (head[1] < 0 or k >= q - head[1]) \
                            and (head[2] < 0 or k <= q + head[2]) and dense[q, k]
                        c += bool(ok)
                want = 0 if c == 0 else (2 if c == bq * bkv else 1)
                assert bm[0, 0, i, j] == want


def test_dense_partial_blocks_closed_forms():
    """Lower-triangular dense mask with square blocks of 32. At S = 256 the
    partial blocks are the 8 diagonal ones, all equal: one distinct mask. At
    S = 250 the last block row is ragged (26 of 32 rows), so its blocks left of
    the diagonal are partial too: 8 diagonal + 7 ragged blocks, with three
    distinct masks (full triangle, ragged triangle, 26 full rows)."""
    blocks, n = oracle.partial_blocks(1, 256, 256, 32, 32, [FULL], np.tri(256, 256, dtype=bool))
    assert sorted(blocks) == [(0, i, i) for i in range(8)] and n == 1
    blocks, n = oracle.partial_blocks(1, 250, 250, 32, 32, [FULL], np.tri(250, 250, dtype=bool))
    assert sorted(blocks) == sorted([(0, i, i) for i in range(8)] + [(0, 7, j) for j in range(7)])
    assert n == 3
    # a per-head stack: head 1 empty, head 0 full -> no partial blocks at all
    d = np.stack([np.ones((64, 64), bool), np.zeros((64, 64), bool)])
    blocks, n = oracle.partial_blocks(2, 64, 64, 16, 16, [FULL], d)
    assert blocks == {} and n == 0


def test_dense_attention_matches_torch_sdpa_fp64():
    """torch's scaled_dot_product_attention with the boolean mask (dense AND
    local window) is a library routine of the same definition."""
    B, H, S, D = 1, 2, 90, 16
    q, k, v, _, _ = _case(23, B, H, S, S, D)
    rng = np.random.default_rng(29)
    dense = rng.random((H, S, S)) < 0.4
    dense[:, np.arange(S), np.arange(S)] = True  # every row keeps a key
    head = (0, 30, 30)
    got = oracle.softmax_attention(q, k, v, 0.25, [head], dense=dense, row_chunk=40)
    for h in range(H):
        m = oracle.element_mask(S, S, head) & dense[h]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, h]), torch.from_numpy(k[0, h]), torch.from_numpy(v[0, h]),
            attn_mask=torch.from_numpy(m), scale=0.25).numpy()
        np.testing.assert_allclose(got[0, h], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# softmax attention
# ---------------------------------------------------------------------------


def _case(seed, B, H, Sq, Skv, D, sigma=1.0, segments=None):
    c = wl.random_case(seed, B, H, Sq, Skv, D, "f32", sigma, segments)
    q, k, v = (_f64(c[n]) for n in ("q", "k", "v"))
    qs = None if c["q_segment_ids"] is None else c["q_segment_ids"].numpy()
    ks = None if c["kv_segment_ids"] is None else c["kv_segment_ids"].numpy()
    return q, k, v, qs, ks


@pytest.mark.parametrize("head", [FULL, CAUSAL, (1, 9, 9), (0, 5, 3)])
@pytest.mark.parametrize("segments", [None, "docs"])
def test_softmax_matches_torch_sdpa_fp64(head, segments):
    """torch's scaled_dot_product_attention in float64 with a boolean mask is a
    library routine of the same definition (rows with no allowed key are
    avoided here: the library returns NaN for them)."""
    B, H, S, D = 2, 3, 97, 32
    q, k, v, qs, ks = _case(11, B, H, S, S, D, segments=segments)
    scale = 1 / math.sqrt(D)
    got = oracle.softmax_attention(q, k, v, scale, [head], qs, ks, row_chunk=40)
    for b in range(B):
        m = oracle.element_mask(S, S, head, None if qs is None else qs[b], None if ks is None else ks[b])
        assert m.any(axis=1).all()
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b]), torch.from_numpy(k[b]), torch.from_numpy(v[b]),
            attn_mask=torch.from_numpy(m), scale=scale).numpy()
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-12)


def test_gqa_head_map_page3_example():
    """Page 3, section 21: 8 query heads over 2 K/V heads, 4 per K/V head."""
    with open(os.path.join(GOLDEN, "page3_sec21_gqa_heads.json")) as f:
        g = json.load(f)
    got = {str(h): oracle.kv_head_of(h, g["q_heads"], g["kv_heads"]) for h in range(g["q_heads"])}
    assert got == g["kv_head_of_q_head"]
    assert g["q_heads"] // g["kv_heads"] == g["q_heads_per_kv_head"]
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)


@pytest.mark.parametrize("kv_heads", [1, 2, 3])
def test_gqa_matches_torch_sdpa_enable_gqa(kv_heads):
    """torch's scaled_dot_product_attention with enable_gqa (K/V heads shared
    by consecutive groups of query heads) is a library routine of the same
    definition."""
    B, H, S, D = 2, 6, 70, 16
    q, _, _, qs, ks = _case(13, B, H, S, S, D, segments="docs")
    rng = np.random.default_rng(7)
    k = rng.standard_normal((B, kv_heads, S, D))
    v = rng.standard_normal((B, kv_heads, S, D))
    scale = 0.3
    got = oracle.softmax_attention(q, k, v, scale, [CAUSAL], qs, ks, row_chunk=32)
    for b in range(B):
        m = oracle.element_mask(S, S, CAUSAL, qs[b], ks[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b]), torch.from_numpy(k[b]), torch.from_numpy(v[b]),
            attn_mask=torch.from_numpy(m), scale=scale, enable_gqa=True).numpy()
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-12)


def test_mqa_identical_query_heads_give_identical_outputs():
    """One K/V head shared by every query head: equal query heads must give
    equal outputs, for softmax and pointwise attention."""
    B, H, S, D = 1, 4, 40, 8
    q, k, v, _, _ = _case(17, B, 1, S, S, D)
    q4 = np.repeat(q, H, axis=1)
    for fn in (oracle.softmax_attention, oracle.pointwise_attention):
        out = fn(q4, k, v, 0.4, [CAUSAL])
        for h in range(1, H):
            assert np.array_equal(out[:, h], out[:, 0])


def test_softmax_closed_forms():
    S, D = 50, 16
    q, k, v, _, _ = _case(3, 1, 1, S, S, D)
    q, k, v = q[0, 0], k[0, 0], v[0, 0]
    mask = oracle.element_mask(S, S, CAUSAL)
    # constant V returns that row
    c = np.linspace(-1, 1, D)
    out = oracle.softmax_attention_rows(q, k, np.tile(c, (S, 1)), 0.3, mask)
    np.testing.assert_allclose(out, np.tile(c, (S, 1)), rtol=0, atol=1e-14)
    # identical keys: the mean of the allowed V rows
    kk = np.tile(k[0], (S, 1))
    out = oracle.softmax_attention_rows(q, kk, v, 0.3, mask)
    want = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-13)
    # scale 0: uniform average of the allowed rows
    out = oracle.softmax_attention_rows(q, k, v, 0.0, mask)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-13)
    # causal row 0 returns v_0 exactly (weight e^0 = 1 over a sum of 1)
    out = oracle.softmax_attention_rows(q, k, v, 0.7, mask)
    assert np.array_equal(out[0], v[0])
    # local window, identical keys: mean over [q - w, q]
    w = 4
    m = oracle.element_mask(S, S, wl.local_causal(w))
    out = oracle.softmax_attention_rows(q, kk, v, 0.3, m)
    want = np.stack([v[max(0, t - w):t + 1].mean(axis=0) for t in range(S)])
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-13)
    # a row with no allowed key returns 0
    m = np.zeros((S, S), dtype=bool)
    assert (oracle.softmax_attention_rows(q, k, v, 0.3, m) == 0).all()


def test_first_token_of_each_document_returns_its_own_value():
    B, H, S, D = 2, 2, 300, 16
    q, k, v, qs, ks = _case(5, B, H, S, S, D, segments="docs")
    out = oracle.softmax_attention(q, k, v, 0.25, [CAUSAL], qs, ks)
    for b in range(B):
        starts = [0] + [t for t in range(1, S) if qs[b, t] != qs[b, t - 1]]
        assert len(starts) > 3
        for t in starts:
            assert np.array_equal(out[b, :, t], v[b, :, t])


def test_softmax_brute_force_scalar_loops():
    """Pure-Python scalar loops with math.exp, S <= 16, random masks."""
    rng = np.random.default_rng(12)
    for trial in range(5):
        Sq, Skv, D = int(rng.integers(1, 17)), int(rng.integers(1, 17)), int(rng.integers(1, 9))
        head = (int(rng.integers(0, 2)), int(rng.integers(-1, 6)), int(rng.integers(-1, 6)))
        q, k, v, qs, ks = _case(100 + trial, 1, 1, Sq, Skv, D, segments="random")
        q, k, v, qs, ks = q[0, 0], k[0, 0], v[0, 0], qs[0], ks[0]
        scale = float(rng.uniform(0.1, 1.0))
        got = oracle.softmax_attention_rows(q, k, v, scale, oracle.element_mask(Sq, Skv, head, qs, ks))
        for t in range(Sq):
            allowed = [j for j in range(Skv)
                       if (not head[0] or j <= t) and (head[1] < 0 or j >= t - head[1])
                       and (head[2] < 0 or j <= t + head[2]) and qs[t] == ks[j]]
            want = [0.0] * D
            if allowed:
                sc = {j: scale * sum(q[t, d] * k[j, d] for d in range(D)) for j in allowed}
                mx = max(sc.values())
                den = sum(math.exp(sc[j] - mx) for j in allowed)
                want = [sum(math.exp(sc[j] - mx) * v[j, d] for j in allowed) / den for d in range(D)]
            np.testing.assert_allclose(got[t], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("block_kv", [1, 3, 7, 16, 64])
def test_online_recurrence_equals_definition(block_kv):
    """Page 3, section 15: the blockwise m, L, O recurrence is exact; the
    result does not depend on the kv block size (page 3, section 14)."""
    S, D = 64, 16
    q, k, v, qs, ks = _case(9, 1, 1, S, S, D, segments="docs")
    for head in (CAUSAL, (1, 10, 10), FULL):
        m = oracle.element_mask(S, S, head, qs[0], ks[0])
        a = oracle.softmax_attention_rows(q[0, 0], k[0, 0], v[0, 0], 0.4, m)
        b = oracle.online_softmax_rows(q[0, 0], k[0, 0], v[0, 0], 0.4, m, block_kv)
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-13)


def test_softmax_large_scores_stay_finite():
    """q x 30 gives |scores| ~ 1e3; the max-subtracted form stays finite and
    agrees with the library routine."""
    S, D = 40, 64
    q, k, v, _, _ = _case(4, 1, 1, S, S, D)
    q = q * 30
    m = oracle.element_mask(S, S, CAUSAL)
    out = oracle.softmax_attention_rows(q[0, 0], k[0, 0], v[0, 0], 0.125, m)
    assert np.isfinite(out).all()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0, 0]), torch.from_numpy(k[0, 0]), torch.from_numpy(v[0, 0]),
        attn_mask=torch.from_numpy(m), scale=0.125).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    b = oracle.online_softmax_rows(q[0, 0], k[0, 0], v[0, 0], 0.125, m, 8)
    np.testing.assert_allclose(b, out, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# pointwise attention
# ---------------------------------------------------------------------------


def test_pointwise_closed_forms():
    S, D = 48, 8
    q, k, v, _, _ = _case(21, 1, 1, S, S, D, sigma=0.5)
    q, k, v = q[0, 0], k[0, 0], v[0, 0]
    mask = oracle.element_mask(S, S, CAUSAL)
    scale = 1 / math.sqrt(D)
    # q = 0: SiLU(0) = 0
    assert (oracle.pointwise_attention_rows(np.zeros_like(q), k, v, scale, mask, S) == 0).all()
    # causal row 0: silu(x) v_0 / S with x = scale <q0, k0>
    out = oracle.pointwise_attention_rows(q, k, v, scale, mask, S)
    x = scale * float(np.dot(q[0], k[0]))
    np.testing.assert_allclose(out[0], x / (1 + math.exp(-x)) * v[0] / S, rtol=1e-14, atol=0)
    # identical keys, constant v = c: |A_q| silu(x_q) c / S
    kk = np.tile(k[3], (S, 1))
    c = np.linspace(-2, 2, D)
    out = oracle.pointwise_attention_rows(q, kk, np.tile(c, (S, 1)), scale, mask, S)
    for t in range(S):
        x = scale * float(np.dot(q[t], k[3]))
        np.testing.assert_allclose(out[t], (t + 1) * x / (1 + math.exp(-x)) * c / S, rtol=1e-12, atol=1e-15)
    # linear in V
    v2 = np.random.default_rng(1).standard_normal(v.shape)
    a = oracle.pointwise_attention_rows(q, k, 2 * v - 3 * v2, scale, mask, S)
    b = 2 * oracle.pointwise_attention_rows(q, k, v, scale, mask, S) \
        - 3 * oracle.pointwise_attention_rows(q, k, v2, scale, mask, S)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_pointwise_brute_force_scalar_loops():
    rng = np.random.default_rng(31)
    for trial in range(5):
        Sq, Skv, D = int(rng.integers(1, 17)), int(rng.integers(1, 17)), int(rng.integers(1, 9))
        head = (int(rng.integers(0, 2)), int(rng.integers(-1, 6)), int(rng.integers(-1, 6)))
        q, k, v, qs, ks = _case(200 + trial, 1, 1, Sq, Skv, D, sigma=0.5, segments="random")
        q, k, v, qs, ks = q[0, 0], k[0, 0], v[0, 0], qs[0], ks[0]
        scale = float(rng.uniform(0.1, 1.0))
        got = oracle.pointwise_attention_rows(q, k, v, scale, oracle.element_mask(Sq, Skv, head, qs, ks), Sq)
        for t in range(Sq):
            want = [0.0] * D
            for j in range(Skv):
                ok = (not head[0] or j <= t) and (head[1] < 0 or j >= t - head[1]) \
                    and (head[2] < 0 or j <= t + head[2]) and qs[t] == ks[j]
                if not ok:
                    continue
                x = scale * sum(q[t, d] * k[j, d] for d in range(D))
                p = x / (1.0 + math.exp(-x)) / Sq
                for d in range(D):
                    want[d] += p * v[j, d]
            np.testing.assert_allclose(got[t], want, rtol=1e-12, atol=1e-15)


def test_full_attention_wrappers_match_rows():
    B, H, S, D = 2, 2, 70, 16
    q, k, v, qs, ks = _case(41, B, H, S, S, D, segments="docs")
    heads = [CAUSAL, wl.local_causal(9)]
    a = oracle.softmax_attention(q, k, v, 0.3, heads, qs, ks, row_chunk=16)
    p = oracle.pointwise_attention(q, k, v, 0.3, heads, qs, ks, row_chunk=16)
    for b in range(B):
        for h in range(H):
            m = oracle.element_mask(S, S, heads[h], qs[b], ks[b])
            np.testing.assert_array_equal(a[b, h], oracle.softmax_attention_rows(q[b, h], k[b, h], v[b, h], 0.3, m))
            np.testing.assert_array_equal(p[b, h], oracle.pointwise_attention_rows(q[b, h], k[b, h], v[b, h], 0.3, m, S))


# ---------------------------------------------------------------------------
# the pins catch planted mistakes
# ---------------------------------------------------------------------------


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible errors in a copy of the oracle's pieces and check that
    the closed forms above reject them."""
    import oracle.splash_oracle as so

    real_allowed = so._allowed

    def off_by_one(qpos, kpos, head):   # window k > q - w instead of k >= q - w
        m = real_allowed(qpos, kpos, head)
        if head[1] >= 0:
            q = np.asarray(qpos)[:, None]
            k = np.asarray(kpos)[None, :]
            m &= k != q - head[1]
        return m

    monkeypatch.setattr(so, "_allowed", off_by_one)
    S, w = 300, 37
    assert so.element_mask(S, S, (1, w, w)).sum() != sum(min(q, w) + 1 for q in range(S))
    monkeypatch.setattr(so, "_allowed", real_allowed)

    # a recurrence without the correction factor alpha disagrees with the definition
    S, D = 64, 16
    q, k, v, _, _ = _case(9, 1, 1, S, S, D)
    m = so.element_mask(S, S, CAUSAL)
    a = so.softmax_attention_rows(q[0, 0], k[0, 0], v[0, 0], 0.4, m)
    real_exp = np.exp
    calls = {"n": 0}

    def exp_without_alpha(x):
        calls["n"] += 1
        if np.ndim(x) == 0:          # the scalar alpha = e^{m_A - m_AB}
            return 1.0
        return real_exp(x)

    monkeypatch.setattr(so.np, "exp", exp_without_alpha)
    b = so.online_softmax_rows(q[0, 0], k[0, 0], v[0, 0], 0.4, m, 8)
    monkeypatch.setattr(so.np, "exp", real_exp)
    assert calls["n"] > 0
    assert not np.allclose(a, b, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------------------
# pointwise backward
# ---------------------------------------------------------------------------


def _loss_grads_fd(q, k, v, do, scale, heads, qs, ks, h=1e-5):
    """Central differences of sum(do * pointwise_attention(q, k, v)) with
    respect to every element of q, k and v (the forward is pinned on its
    own above)."""
    def loss(qq, kk, vv):
        return float((oracle.pointwise_attention(qq, kk, vv, scale, heads, qs, ks) * do).sum())

    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(g.shape):
            x0 = args[which][idx]
            args[which][idx] = x0 + h
            up = loss(*args)
            args[which][idx] = x0 - h
            dn = loss(*args)
            args[which][idx] = x0
            g[idx] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


def _small_bwd_case(seed, H, kv_heads, Sq, Skv, D):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, H, Sq, D))
    k = rng.standard_normal((1, kv_heads, Skv, D))
    v = rng.standard_normal((1, kv_heads, Skv, D))
    do = rng.standard_normal((1, H, Sq, D))
    qs = rng.integers(0, 2, size=(1, Sq)).astype(np.int32)
    ks = rng.integers(0, 2, size=(1, Skv)).astype(np.int32)
    return q, k, v, do, qs, ks


@pytest.mark.parametrize("kv_heads", [2, 1])
def test_pointwise_bwd_matches_finite_differences(kv_heads):
    """The gradients are those of the (separately pinned) forward: central
    differences of sum(do * out), every element of q, k and v, with head masks,
    segment ids and (kv_heads = 1) two query heads sharing one K/V head."""
    H, Sq, Skv, D = 2, 7, 9, 3
    q, k, v, do, qs, ks = _small_bwd_case(5 + kv_heads, H, kv_heads, Sq, Skv, D)
    heads = [CAUSAL, (0, 2, 3)]
    dq, dk, dv = oracle.pointwise_attention_bwd(q, k, v, do, 0.7, heads, qs, ks, row_chunk=3)
    fq, fk, fv = _loss_grads_fd(q, k, v, do, 0.7, heads, qs, ks)
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(want).max() > 1e-3
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-8)


@pytest.mark.parametrize("head", [FULL, CAUSAL, (1, 9, 9), (0, 5, 3)])
def test_pointwise_bwd_matches_torch_autograd(head):
    """torch autograd through torch's own SiLU (a library derivative) in
    float64: out = silu(scale q k^T) / Sq, masked to 0, times v."""
    B, H, S, D = 2, 2, 61, 16
    q, k, v, qs, ks = _case(71, B, H, S, S, D, sigma=0.8, segments="docs")
    do = np.random.default_rng(72).standard_normal(q.shape)
    scale = 1 / math.sqrt(D)
    dq, dk, dv = oracle.pointwise_attention_bwd(q, k, v, do, scale, [head], qs, ks, row_chunk=20)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    total = 0
    for b in range(B):
        m = torch.from_numpy(oracle.element_mask(S, S, head, qs[b], ks[b]))
        x = scale * (tq[b] @ tk[b].transpose(-1, -2))
        p = torch.where(m, torch.nn.functional.silu(x), torch.zeros((), dtype=torch.float64)) / S
        total = total + ((p @ tv[b]) * torch.from_numpy(do[b])).sum()
    total.backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_pointwise_bwd_closed_forms():
    S, D = 40, 8
    q, k, v, _, _ = _case(73, 1, 1, S, S, D, sigma=0.6)
    do = np.random.default_rng(74).standard_normal(q.shape)
    scale = 0.35
    mask = oracle.element_mask(S, S, CAUSAL)
    q0, k0, v0, do0 = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    # do = 0: nothing flows back
    for g in oracle.pointwise_attention_bwd_rows(q0, k0, v0, np.zeros_like(do0), scale, mask, S):
        assert (g == 0).all()
    # v = 0: dp = 0, so dq = dk = 0; dv = P^T do with P the forward's weights
    # (the forward with v = identity returns P itself)
    dq, dk, dv = oracle.pointwise_attention_bwd_rows(q0, k0, np.zeros_like(v0), do0, scale, mask, S)
    assert (dq == 0).all() and (dk == 0).all()
    P = oracle.pointwise_attention_rows(q0, k0, np.eye(S), scale, mask, S)
    np.testing.assert_allclose(dv, P.T @ do0, rtol=1e-12, atol=1e-15)
    # q = 0: every score is 0, silu'(0) = 1/2, silu(0) = 0:
    # dv = 0, dk = 0, dq_t = scale / (2 S) sum_{k <= t} (do_t . v_k) k_k
    dq, dk, dv = oracle.pointwise_attention_bwd_rows(np.zeros_like(q0), k0, v0, do0, scale, mask, S)
    assert (dv == 0).all() and (dk == 0).all()
    for t in range(S):
        want = sum(float(np.dot(do0[t], v0[j])) * k0[j] for j in range(t + 1)) * scale / (2 * S)
        np.testing.assert_allclose(dq[t], want, rtol=1e-12, atol=1e-15)
    # causal: the last key is seen only by the last query
    dq, dk, dv = oracle.pointwise_attention_bwd_rows(q0, k0, v0, do0, scale, mask, S)
    x = scale * float(np.dot(q0[S - 1], k0[S - 1]))
    sig = 1 / (1 + math.exp(-x))
    np.testing.assert_allclose(dv[S - 1], x * sig / S * do0[S - 1], rtol=1e-12, atol=0)
    ds = float(np.dot(do0[S - 1], v0[S - 1])) * sig * (1 + x * (1 - sig)) / S
    np.testing.assert_allclose(dk[S - 1], scale * ds * q0[S - 1], rtol=1e-12, atol=0)


def test_pointwise_bwd_masked_keys_get_no_gradient():
    """Keys that no query may see get dk = dv = 0, and changing them leaves dq
    unchanged (documents: a key whose id no query has)."""
    B, H, S, D = 1, 2, 50, 8
    q, k, v, qs, ks = _case(75, B, H, S, S, D)
    do = np.random.default_rng(76).standard_normal(q.shape)
    qs = np.zeros((1, S), np.int32)
    ks = np.zeros((1, S), np.int32)
    ks[0, 10:20] = 7
    dq, dk, dv = oracle.pointwise_attention_bwd(q, k, v, do, 0.5, [FULL], qs, ks)
    assert (dk[0, :, 10:20] == 0).all() and (dv[0, :, 10:20] == 0).all()
    assert np.abs(dk[0, :, :10]).min() > 0
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 10:20] += 3.0
    v2[0, :, 10:20] -= 1.0
    dq2, _, _ = oracle.pointwise_attention_bwd(q, k2, v2, do, 0.5, [FULL], qs, ks)
    np.testing.assert_array_equal(dq, dq2)


def test_pointwise_bwd_pins_catch_planted_mistakes(monkeypatch):
    """Mutants of the backward (a dropped term, a lost scale, an unmasked
    sigmoid, a missing 1/seq_len) all fail the finite-difference pin."""
    import inspect
    import oracle.splash_oracle as so

    H, Sq, Skv, D = 2, 6, 6, 3
    q, k, v, do, qs, ks = _small_bwd_case(77, H, 2, Sq, Skv, D)
    heads = [CAUSAL]
    fd = _loss_grads_fd(q, k, v, do, 0.6, heads, qs, ks)
    src = inspect.getsource(so.pointwise_attention_bwd_rows)
    mutations = [
        ("* (1.0 + qk * (1.0 - sig))", "* (qk * (1.0 - sig))"),
        ("dk = float(scale) * (ds @ q_rows)", "dk = ds @ q_rows"),
        ("sig = np.where(np.asarray(mask_rows).T, _logistic(qk), 0.0)", "sig = _logistic(qk)"),
        ("ds = dp * sig * (1.0 + qk * (1.0 - sig)) / float(seq_len)", "ds = dp * sig * (1.0 + qk * (1.0 - sig))"),
    ]
    for old, new in mutations:
        assert old in src, old
        ns = dict(so.__dict__)
        exec(src.replace(old, new), ns)
        monkeypatch.setattr(so, "pointwise_attention_bwd_rows", ns["pointwise_attention_bwd_rows"])
        got = so.pointwise_attention_bwd(q, k, v, do, 0.6, heads, qs, ks)
        err = max(np.abs(g - f).max() for g, f in zip(got, fd))
        assert err > 1e-4, (old, err)
    monkeypatch.undo()
    got = so.pointwise_attention_bwd(q, k, v, do, 0.6, heads, qs, ks)
    assert max(np.abs(g - f).max() for g, f in zip(got, fd)) < 1e-8


def test_dkv_metadata_closed_forms_and_brute_force():
    """Column walk of the dK/dV pass: causal square blocks give
    data_next[i, j] = max(i, j) (column j is non-empty from q block j on);
    every case matches a scalar scan down each column, and the classes are
    the forward's."""
    S, b = 1000, 64
    nq = -(-S // b)
    bm, dn = oracle.mask_info_dkv(1, 1, S, S, b, b, [CAUSAL])
    for i in range(nq):
        for j in range(nq):
            assert dn[0, 0, i, j] == max(i, j)
    rng = np.random.default_rng(78)
    for trial in range(6):
        Sq, Skv = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        bq, bkv = int(rng.choice([16, 32, 64])), int(rng.choice([16, 32, 64]))
        heads = [(int(rng.integers(0, 2)), int(rng.integers(-1, 40)), int(rng.integers(-1, 40))) for _ in range(2)]
        _, _, _, qs, ks = _case(300 + trial, 2, 1, Sq, Skv, 4, segments="random")
        fbm, _ = oracle.mask_info(2, 2, Sq, Skv, bq, bkv, heads, qs, ks)
        bm, dn = oracle.mask_info_dkv(2, 2, Sq, Skv, bq, bkv, heads, qs, ks)
        np.testing.assert_array_equal(bm, fbm)
        Bm, Hm, nq, nk = bm.shape
        for bb in range(Bm):
            for h in range(Hm):
                for j in range(nk):
                    for i in range(nq):
                        later = [ii for ii in range(i, nq) if bm[bb, h, ii, j] != 0]
                        assert dn[bb, h, i, j] == (later[0] if later else nq)


# ---------------------------------------------------------------------------
# softmax log-sum-exp and backward
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("head", [FULL, CAUSAL, (1, 9, 9), (0, 5, 3)])
def test_softmax_lse_matches_torch_logsumexp(head):
    """torch.logsumexp (a library routine) over the allowed scores; rows with
    no allowed key give -inf."""
    B, H, S, D = 2, 2, 70, 16
    q, k, v, qs, ks = _case(81, B, H, S, S, D, segments="docs")
    got = oracle.softmax_lse(q, k, 0.3, [head], qs, ks)
    for b in range(B):
        m = torch.from_numpy(oracle.element_mask(S, S, head, qs[b], ks[b]))
        for h in range(H):
            a = 0.3 * torch.from_numpy(q[b, h]) @ torch.from_numpy(k[b, h]).T
            want = torch.logsumexp(a.masked_fill(~m, float("-inf")), dim=1).numpy()
            np.testing.assert_allclose(got[b, h], want, rtol=1e-13, atol=1e-13)
    # identical keys: log(n e^x) = x + log n, n = allowed keys of the row
    kk = np.tile(k[0, 0, 3], (S, 1))
    lse = oracle.softmax_lse_rows(q[0, 0], kk, 0.3, oracle.element_mask(S, S, CAUSAL))
    for t in range(S):
        x = 0.3 * float(np.dot(q[0, 0, t], k[0, 0, 3]))
        assert abs(lse[t] - (x + math.log(t + 1))) < 1e-12
    # no allowed key
    none = oracle.softmax_lse_rows(q[0, 0, :2], k[0, 0], 1.0, np.zeros((2, S), bool))
    assert (none == -np.inf).all()


@pytest.mark.parametrize("head", [FULL, CAUSAL, (1, 9, 9), (0, 5, 3)])
def test_softmax_bwd_matches_torch_sdpa_autograd(head):
    """Autograd through torch's scaled_dot_product_attention in float64 (a
    library definition and derivative) with a boolean mask."""
    B, H, S, D = 2, 2, 61, 16
    q, k, v, qs, ks = _case(83, B, H, S, S, D, segments="docs")
    do = np.random.default_rng(84).standard_normal(q.shape)
    scale = 1 / math.sqrt(D)
    dq, dk, dv = oracle.softmax_attention_bwd(q, k, v, do, scale, [head], qs, ks, row_chunk=25)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    total = 0
    for b in range(B):
        m = torch.from_numpy(oracle.element_mask(S, S, head, qs[b], ks[b]))
        assert m.any(dim=1).all()
        o = torch.nn.functional.scaled_dot_product_attention(tq[b], tk[b], tv[b], attn_mask=m, scale=scale)
        total = total + (o * torch.from_numpy(do[b])).sum()
    total.backward()
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("kv_heads", [2, 1])
def test_softmax_bwd_matches_finite_differences(kv_heads):
    """Central differences of sum(do * softmax_attention) (the forward is
    pinned above), with head masks, segment ids and a shared K/V head."""
    H, Sq, Skv, D = 2, 7, 9, 3
    q, k, v, do, qs, ks = _small_bwd_case(85 + kv_heads, H, kv_heads, Sq, Skv, D)
    heads = [CAUSAL, (0, 2, 3)]
    qs[:] = 0
    ks[:] = 0
    ks[0, ::3] = 1   # some keys in another document
    dq, dk, dv = oracle.softmax_attention_bwd(q, k, v, do, 0.7, heads, qs, ks, row_chunk=3)

    def loss(qq, kk, vv):
        return float((oracle.softmax_attention(qq, kk, vv, 0.7, heads, qs, ks) * do).sum())

    for which, got in enumerate((dq, dk, dv)):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(g.shape):
            x0 = args[which][idx]
            args[which][idx] = x0 + 1e-5
            up = loss(*args)
            args[which][idx] = x0 - 1e-5
            dn = loss(*args)
            args[which][idx] = x0
            g[idx] = (up - dn) / 2e-5
        assert np.abs(g).max() > 1e-3
        np.testing.assert_allclose(got, g, rtol=0, atol=1e-8)


def test_softmax_bwd_closed_forms_and_mutants(monkeypatch):
    """v constant: every row's output is that constant whatever the scores,
    so dq = dk = 0 and dv = P^T do (P from the forward with v = identity).
    Mutants (delta dropped, scale lost) fail the closed forms or torch."""
    import inspect
    import oracle.splash_oracle as so

    S, D = 40, 8
    q, k, v, _, _ = _case(87, 1, 1, S, S, D)
    do = np.random.default_rng(88).standard_normal((S, D))
    mask = oracle.element_mask(S, S, CAUSAL)
    c = np.linspace(-1, 1, D)
    dq, dk, dv = oracle.softmax_attention_bwd_rows(q[0, 0], k[0, 0], np.tile(c, (S, 1)), do, 0.4, mask)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    P = oracle.softmax_attention_rows(q[0, 0], k[0, 0], np.eye(S), 0.4, mask)
    np.testing.assert_allclose(dv, P.T @ do, rtol=1e-12, atol=1e-14)
    # a row with no allowed key contributes nothing
    none = np.zeros((2, S), bool)
    for g in oracle.softmax_attention_bwd_rows(q[0, 0, :2], k[0, 0], v[0, 0], do[:2], 0.4, none):
        assert (g == 0).all()

    src = inspect.getsource(so.softmax_attention_bwd_rows)
    ref = oracle.softmax_attention_bwd_rows(q[0, 0], k[0, 0], v[0, 0], do, 0.4, mask)
    for old, new in [("dS = P * (dP - delta)", "dS = P * dP"),
                     ("dq = float(scale) * (dS @ k)", "dq = dS @ k"),
                     ("dv = P.T @ do_rows", "dv = P @ do_rows")]:
        assert old in src
        ns = dict(so.__dict__)
        exec(src.replace(old, new), ns)
        got = ns["softmax_attention_bwd_rows"](q[0, 0], k[0, 0], v[0, 0], do, 0.4, mask)
        err = max(np.abs(a - b).max() for a, b in zip(got, ref))
        # the real function is pinned to torch above; a mutant moves away from it
        assert err > 1e-3, old


# ---------------------------------------------------------------------------
# backward under dense masks
# ---------------------------------------------------------------------------


def _torch_mask(S, head, dense_h, qs_b, ks_b):
    """Boolean [S, S] element mask built with torch from the definitions:
    causal k <= q, window q - wl <= k <= q + wr, the dense array's bit, and
    segment equality."""
    causal, wl_, wr = head
    qp = torch.arange(S)[:, None]
    kp = torch.arange(S)[None, :]
    m = torch.ones(S, S, dtype=torch.bool)
    if causal:
        m &= kp <= qp
    if wl_ >= 0:
        m &= kp >= qp - wl_
    if wr >= 0:
        m &= kp <= qp + wr
    m &= torch.from_numpy(dense_h)
    m &= torch.from_numpy(qs_b)[:, None] == torch.from_numpy(ks_b)[None, :]
    return m


@pytest.mark.parametrize("head", [FULL, CAUSAL, (0, 5, 3)])
def test_dense_bwd_matches_torch_autograd(head):
    """The backwards with a per-head dense mask (and segment ids) against
    torch autograd in float64: softmax through scaled_dot_product_attention
    with the boolean mask, pointwise through torch's SiLU masked to 0."""
    B, H, S, D = 2, 2, 53, 16
    q, k, v, qs, ks = _case(91, B, H, S, S, D, sigma=0.8, segments="docs")
    rng = np.random.default_rng(92)
    dense = rng.random((H, S, S)) < 0.6
    dense[:, np.arange(S), np.arange(S)] = True  # every row keeps a key
    do = rng.standard_normal(q.shape)
    scale = 1 / math.sqrt(D)
    for kind in ("softmax", "pointwise"):
        fn = oracle.softmax_attention_bwd if kind == "softmax" else oracle.pointwise_attention_bwd
        dq, dk, dv = fn(q, k, v, do, scale, [head], qs, ks, row_chunk=20, dense=dense)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        total = 0
        for b in range(B):
            for h in range(H):
                m = _torch_mask(S, head, dense[h], qs[b], ks[b])
                if kind == "softmax":
                    o = torch.nn.functional.scaled_dot_product_attention(
                        tq[b, h][None], tk[b, h][None], tv[b, h][None], attn_mask=m, scale=scale)[0]
                else:
                    x = scale * (tq[b, h] @ tk[b, h].T)
                    p = torch.where(m, torch.nn.functional.silu(x), torch.zeros((), dtype=torch.float64)) / S
                    o = p @ tv[b, h]
                total = total + (o * torch.from_numpy(do[b, h])).sum()
        total.backward()
        for got, t in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=kind)
    # the log-sum-exp under the same mask against torch.logsumexp
    lse = oracle.softmax_lse(q, k, scale, [head], qs, ks, dense=dense)
    for b in range(B):
        for h in range(H):
            m = _torch_mask(S, head, dense[h], qs[b], ks[b])
            x = scale * torch.from_numpy(q[b, h]) @ torch.from_numpy(k[b, h]).T
            want = torch.logsumexp(x.masked_fill(~m, -math.inf), dim=-1).numpy()
            np.testing.assert_allclose(lse[b, h], want, rtol=1e-12, atol=1e-12)


def test_dense_bwd_lower_triangle_is_causal_and_dropped_mask_fails():
    """A lower-triangular dense mask under the full head mask gives the causal
    gradients; a dense mask that the backward ignored would not."""
    B, H, S, D = 1, 2, 47, 8
    q, k, v, _, _ = _case(93, B, H, S, S, D)
    do = np.random.default_rng(94).standard_normal(q.shape)
    tri = np.tri(S, S, dtype=bool)
    for fn in (oracle.softmax_attention_bwd, oracle.pointwise_attention_bwd):
        a = fn(q, k, v, do, 0.3, [FULL], dense=tri)
        c = fn(q, k, v, do, 0.3, [CAUSAL])
        f = fn(q, k, v, do, 0.3, [FULL])
        for x, y, z in zip(a, c, f):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)
            assert not np.allclose(x, z)
