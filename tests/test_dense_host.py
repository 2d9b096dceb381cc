"""The library's host-side dense-mask metadata builder against the oracle.

splash_dense_mask_info_host runs on the CPU, so these tests call it through
the C ABI with numpy buffers and need no GPU. Block classes and data_next are
compared bit for bit; the store of partial blocks is unique only up to the
order of its entries, so every partial block's entry is unpacked and compared
with the oracle's element mask of that block, and the number of entries with
the oracle's count of distinct partial blocks.
"""

import ctypes

import numpy as np
import pytest

import oracle
from block_sparse_masked_splash_amd import binding as bd

CAUSAL, FULL = (1, -1, -1), (0, -1, -1)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def build(dense, heads, bq, bkv, capacity=None):
    lib = bd.load_library()
    dense = np.ascontiguousarray(dense, dtype=np.uint8)
    if dense.ndim == 2:
        dense = dense[None]
    Hd, Sq, Skv = dense.shape
    arr, nmh = bd._head_array(heads)
    hp = ctypes.cast(arr, ctypes.POINTER(bd.HeadMaskC))
    Hm = max(Hd, nmh)
    nq, nk = -(-Sq // bq), -(-Skv // bkv)
    n = ctypes.c_int64(-1)
    st = lib.splash_dense_mask_info_host(Sq, Skv, bq, bkv, nmh, hp, Hd, _ptr(dense), Hm, None, None, None, None, 0,
                                         ctypes.byref(n))
    assert st == bd.SPLASH_OK, lib.splash_last_error()
    count = n.value
    bm = np.full((Hm, nq, nk), -7, dtype=np.int8)
    dn = np.full((Hm, nq, nk), -7, dtype=np.int32)
    mn = np.full((Hm, nq, nk), -7, dtype=np.int32)
    cap = count if capacity is None else capacity
    blocks = np.zeros((max(cap, 1), bq, bkv // 32), dtype=np.uint32)
    st = lib.splash_dense_mask_info_host(Sq, Skv, bq, bkv, nmh, hp, Hd, _ptr(dense), Hm, _ptr(bm), _ptr(dn), _ptr(mn),
                                         _ptr(blocks), cap, ctypes.byref(n))
    return st, bm, dn, mn, blocks[:count], count


def unpack(entry, bkv):
    """[bq, bkv/32] words -> boolean [bq, bkv]: bit b of word w is key 32 w + b."""
    bits = (entry[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(entry.shape[0], bkv).astype(bool)


CASES = [
    # Sq, Skv, bq, bkv, number of dense heads, head masks, density
    (256, 256, 64, 64, 1, [FULL], "tril"),
    (250, 250, 64, 64, 1, [FULL], "tril"),
    (300, 420, 128, 128, 1, [CAUSAL], 0.5),
    (200, 160, 64, 128, 3, [FULL], 0.1),
    (333, 333, 128, 64, 2, [CAUSAL, (0, 40, 40)], 0.9),
    (130, 257, 32, 32, 1, [(1, 20, 20)], 0.6),
    (97, 64, 16, 64, 4, [FULL, CAUSAL, (0, 5, 5), (1, 30, 30)], 0.3),
]


@pytest.mark.parametrize("case", CASES, ids=[f"d{n}" for n in range(len(CASES))])
def test_dense_host_metadata_matches_oracle(case):
    Sq, Skv, bq, bkv, Hd, heads, density = case
    rng = np.random.default_rng(hash(case[:5]) % 2**32)
    if density == "tril":
        dense = np.tri(Sq, Skv, dtype=bool)[None].repeat(Hd, axis=0)
    else:
        dense = rng.random((Hd, Sq, Skv)) < density
    H = max(Hd, len(heads))
    st, bm, dn, mn, blocks, count = build(dense, heads, bq, bkv)
    assert st == bd.SPLASH_OK
    obm, odn = oracle.mask_info(1, H, Sq, Skv, bq, bkv, heads, dense=dense)
    np.testing.assert_array_equal(bm, obm[0])
    np.testing.assert_array_equal(dn, odn[0])
    oblocks, distinct = oracle.partial_blocks(H, Sq, Skv, bq, bkv, heads, dense)
    assert count == distinct
    assert ((mn == 0) | (bm == 1)).all()          # only partial blocks name an entry
    assert sorted(map(tuple, np.argwhere(bm == 1))) == sorted(oblocks)
    for (hm, i, j), want in oblocks.items():
        m = mn[hm, i, j]
        assert 0 <= m < count
        np.testing.assert_array_equal(unpack(blocks[m], bkv), want, err_msg=str((hm, i, j)))
    # minimal store: every entry is used and no two entries are equal
    assert sorted(set(mn[bm == 1].tolist())) == list(range(count))
    assert len({blocks[n].tobytes() for n in range(count)}) == count


def test_dense_host_causal_store_is_one_triangle():
    """A causal dense mask with square blocks that divide the length: every
    diagonal block is the same lower triangle, so the store has one entry."""
    S, b = 512, 64
    st, bm, dn, mn, blocks, count = build(np.tri(S, S, dtype=bool), [FULL], b, b)
    assert st == bd.SPLASH_OK and count == 1
    np.testing.assert_array_equal(unpack(blocks[0], b), np.tri(b, b, dtype=bool))


def test_dense_host_errors():
    lib = bd.load_library()
    dense = np.ones((1, 64, 64), dtype=np.uint8)
    arr, nmh = bd._head_array([FULL])
    hp = ctypes.cast(arr, ctypes.POINTER(bd.HeadMaskC))
    n = ctypes.c_int64(0)
    out = [np.zeros((1, 1, 1), dtype=t) for t in (np.int8, np.int32, np.int32)]

    def call(bq=64, bkv=64, Hd=1, Hm=1, cap=4, dense_p=_ptr(dense)):
        return lib.splash_dense_mask_info_host(64, 64, bq, bkv, nmh, hp, Hd, dense_p, Hm, *map(_ptr, out),
                                               _ptr(np.zeros(64 * 4, np.uint32)), cap, ctypes.byref(n))

    assert call(bkv=48) == bd.SPLASH_ERR_INVALID_ARGUMENT      # block_kv not a multiple of 32
    assert b"multiple of 32" in lib.splash_last_error()
    assert call(Hm=2) == bd.SPLASH_ERR_INVALID_ARGUMENT        # meta_heads not max(heads)
    assert call(dense_p=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(cap=-1) == bd.SPLASH_ERR_INVALID_ARGUMENT
    # a store too small: error, nothing written
    d = np.tri(128, 128, dtype=np.uint8)[None]
    st, bm, *_ = build(d, [FULL], 32, 32, capacity=0)
    assert st == bd.SPLASH_ERR_INVALID_ARGUMENT and (bm == -7).all()
    assert b"capacity" in lib.splash_last_error()


def build_ex(dense, heads, bq, bkv, B=1, q_seg=None, kv_seg=None, columns=0):
    """splash_dense_mask_info_host_ex: (status, block_mask, data_next,
    mask_next, store, count), arrays [Bm, Hm, nq, nk] (columns: [.., nk, nq])."""
    lib = bd.load_library()
    dense = np.ascontiguousarray(dense, dtype=np.uint8)
    if dense.ndim == 2:
        dense = dense[None]
    Hd, Sq, Skv = dense.shape
    arr, nmh = bd._head_array(heads)
    hp = ctypes.cast(arr, ctypes.POINTER(bd.HeadMaskC))
    Hm = max(Hd, nmh)
    Bm = B if q_seg is not None else 1
    qs = None if q_seg is None else np.ascontiguousarray(q_seg, dtype=np.int32)
    ks = None if kv_seg is None else np.ascontiguousarray(kv_seg, dtype=np.int32)
    nq, nk = -(-Sq // bq), -(-Skv // bkv)
    n = ctypes.c_int64(-1)
    st = lib.splash_dense_mask_info_host_ex(B, Sq, Skv, bq, bkv, nmh, hp, Hd, _ptr(dense), Hm, _ptr(qs), _ptr(ks),
                                            columns, None, None, None, None, 0, ctypes.byref(n))
    assert st == bd.SPLASH_OK, lib.splash_last_error()
    count = n.value
    shape = (Bm, Hm, nk, nq) if columns else (Bm, Hm, nq, nk)
    bm = np.full(shape, -7, dtype=np.int8)
    dn = np.full(shape, -7, dtype=np.int32)
    mn = np.full(shape, -7, dtype=np.int32)
    blocks = np.zeros((max(count, 1), bq, bkv // 32), dtype=np.uint32)
    st = lib.splash_dense_mask_info_host_ex(B, Sq, Skv, bq, bkv, nmh, hp, Hd, _ptr(dense), Hm, _ptr(qs), _ptr(ks),
                                            columns, _ptr(bm), _ptr(dn), _ptr(mn), _ptr(blocks), count,
                                            ctypes.byref(n))
    return st, bm, dn, mn, blocks[:count], count


EX_CASES = [
    # B, Sq, Skv, bq, bkv, dense heads, head masks, density, segments, columns
    (2, 300, 300, 64, 64, 1, [CAUSAL], "tril", "docs", 0),
    (3, 250, 250, 128, 64, 2, [FULL, CAUSAL], 0.7, "docs", 0),
    (2, 200, 230, 64, 128, 1, [(1, 40, 40)], 0.5, "random", 0),
    (1, 300, 260, 96, 64, 1, [CAUSAL], 0.6, None, 1),
    (2, 333, 333, 64, 128, 2, [CAUSAL, (0, 30, 30)], "tril", "docs", 1),
    (2, 150, 190, 32, 64, 1, [FULL], 0.4, "random", 1),
]


@pytest.mark.parametrize("case", EX_CASES, ids=[f"x{n}" for n in range(len(EX_CASES))])
def test_dense_host_segments_and_columns_match_oracle(case):
    """Segment ids folded into the classes and bits (one metadata batch row
    per batch row), and the dK/dV walk's column layout: classes, data_next
    and every partial block's entry against the oracle."""
    B, Sq, Skv, bq, bkv, Hd, heads, density, seg, columns = case
    rng = np.random.default_rng(sum(case[:5]) + columns)
    if density == "tril":
        dense = np.tri(Sq, Skv, dtype=bool)[None].repeat(Hd, axis=0)
    else:
        dense = rng.random((Hd, Sq, Skv)) < density
    qs = ks = None
    if seg == "docs":
        from block_sparse_masked_splash_amd import workloads as wl
        qs = wl.draw_documents(rng, B, Sq, 1, 90)
        ks = qs if Skv == Sq else wl.draw_documents(rng, B, Skv, 1, 90)
    elif seg == "random":
        qs = rng.integers(0, 3, size=(B, Sq)).astype(np.int32)
        ks = rng.integers(0, 3, size=(B, Skv)).astype(np.int32)
    H = max(Hd, len(heads))
    st, bm, dn, mn, blocks, count = build_ex(dense, heads, bq, bkv, B, qs, ks, columns)
    assert st == bd.SPLASH_OK
    if columns:
        obm, odn = oracle.mask_info_dkv(B, H, Sq, Skv, bq, bkv, heads, qs, ks, dense=dense)
        obm, odn = obm.transpose(0, 1, 3, 2), odn.transpose(0, 1, 3, 2)
    else:
        obm, odn = oracle.mask_info(B, H, Sq, Skv, bq, bkv, heads, qs, ks, dense=dense)
    np.testing.assert_array_equal(bm, obm)
    np.testing.assert_array_equal(dn, odn)
    assert ((mn == 0) | (bm == 1)).all()
    seen = set()
    for b in range(bm.shape[0]):
        for hm in range(bm.shape[1]):
            head = heads[0] if len(heads) == 1 else heads[hm]
            dm = dense[0] if Hd == 1 else dense[hm]
            qb = None if qs is None else qs[b]
            kb = None if ks is None else ks[b]
            for i in range(-(-Sq // bq)):
                pm = oracle.padded_element_mask(Sq, Skv, bq, bkv, head, qb, kb, q_block=i, dense=dm)
                for j in range(-(-Skv // bkv)):
                    c = bm[b, hm, j, i] if columns else bm[b, hm, i, j]
                    if c != 1:
                        continue
                    m = mn[b, hm, j, i] if columns else mn[b, hm, i, j]
                    want = pm[:, j * bkv:(j + 1) * bkv]
                    np.testing.assert_array_equal(unpack(blocks[m], bkv), want, err_msg=str((b, hm, i, j)))
                    seen.add(want.tobytes())
    assert count == len(seen)                      # one entry per distinct partial block
    assert len({blocks[n].tobytes() for n in range(count)}) == count


def test_dense_host_ex_errors_and_plain_form():
    """The plain builder is the extended one with B = 1, no segment ids and
    rows; one segment array without the other and a bad layout flag are
    refused."""
    rng = np.random.default_rng(3)
    dense = rng.random((1, 200, 200)) < 0.5
    a = build(dense, [CAUSAL], 64, 64)
    b = build_ex(dense, [CAUSAL], 64, 64)
    for x, y in zip(a[1:4], b[1:4]):
        np.testing.assert_array_equal(x, y[0])
    np.testing.assert_array_equal(a[4], b[4])
    lib = bd.load_library()
    d = np.ascontiguousarray(dense, dtype=np.uint8)
    arr, nmh = bd._head_array([FULL])
    hp = ctypes.cast(arr, ctypes.POINTER(bd.HeadMaskC))
    n = ctypes.c_int64(0)
    ids = np.zeros((1, 200), np.int32)
    assert lib.splash_dense_mask_info_host_ex(1, 200, 200, 64, 64, nmh, hp, 1, _ptr(d), 1, _ptr(ids), None, 0,
                                              None, None, None, None, 0, ctypes.byref(n)) == \
        bd.SPLASH_ERR_INVALID_ARGUMENT
    assert lib.splash_dense_mask_info_host_ex(1, 200, 200, 64, 64, nmh, hp, 1, _ptr(d), 1, None, None, 2,
                                              None, None, None, None, 0, ctypes.byref(n)) == \
        bd.SPLASH_ERR_INVALID_ARGUMENT
    assert lib.splash_dense_mask_info_host_ex(-1, 200, 200, 64, 64, nmh, hp, 1, _ptr(d), 1, None, None, 0,
                                              None, None, None, None, 0, ctypes.byref(n)) == \
        bd.SPLASH_ERR_INVALID_ARGUMENT
