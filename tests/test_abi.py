"""C ABI checks that need no GPU: exports, version, and argument validation.

Every call made here fails validation on the host, which by contract happens
before any HIP call, so nothing touches a device.
"""

import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_masked_splash_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "splash.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(splash_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert set(declared) == set(bd.SYMBOLS)
    lib = bd.load_library()
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", bd.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (splash_\w+)", out))
    assert set(declared) <= exported


def test_version_and_status_strings():
    lib = bd.load_library()
    assert lib.splash_abi_version() == 1
    assert lib.splash_status_string(0) == b"SPLASH_OK"
    assert lib.splash_status_string(3) == b"SPLASH_ERR_METADATA_MISMATCH"
    assert lib.splash_status_string(99) == b"SPLASH_ERR_UNKNOWN"


def _desc(heads=((1, -1, -1),), qseg=None, kvseg=None, n=None):
    arr, cnt = bd._head_array(heads)
    d = bd.MaskDescC(cnt if n is None else n, ctypes.cast(arr, ctypes.POINTER(bd.HeadMaskC)), qseg, kvseg)
    return d, arr


def test_mask_info_entries():
    lib = bd.load_library()
    d, keep = _desc()
    assert lib.splash_mask_info_entries(2, 4, 256, 256, 64, 64, ctypes.byref(d)) == 16
    assert lib.splash_mask_info_entries(2, 4, 200, 130, 64, 64, ctypes.byref(d)) == 4 * 3
    d2, keep2 = _desc(qseg=0x1000, kvseg=0x2000)
    assert lib.splash_mask_info_entries(2, 4, 256, 256, 64, 64, ctypes.byref(d2)) == 2 * 16
    d3, keep3 = _desc(qseg=0x1000)
    assert lib.splash_mask_info_entries(2, 4, 256, 256, 64, 64, ctypes.byref(d3)) == 0
    assert lib.splash_mask_info_entries(2, 4, 256, 256, 0, 64, ctypes.byref(d)) == 0
    assert lib.splash_mask_info_entries(2, 4, -1, 256, 64, 64, ctypes.byref(d)) == 0
    d4, keep4 = _desc(heads=[(1, -1, -1)] * 3)
    assert lib.splash_mask_info_entries(2, 4, 256, 256, 64, 64, ctypes.byref(d4)) == 0


def _info(Bm=1, Hm=1, nq=4, nk=4, bq=64, bkv=64, bm=0x10000, dn=0x20000):
    return bd.MaskInfoC(Bm, Hm, nq, nk, bq, bkv, bm, dn)


def _fwd(lib, fn="splash_fwd", in_dt=1, out_dt=1, B=1, H=1, Sq=256, Skv=256, D=128, q=0x100000,
         k=0x200000, v=0x300000, o=0x400000, strides=None, scale=0.1, desc=None, info=None):
    st = strides or [bd._I64x3(H * Sq * D, Sq * D, D) for _ in range(4)]
    return getattr(lib, fn)(in_dt, out_dt, B, H, Sq, Skv, D, q, st[0], k, st[1], v, st[2], o, st[3],
                            scale, None if desc is None else ctypes.byref(desc),
                            None if info is None else ctypes.byref(info), None)


@pytest.mark.parametrize("fn", ["splash_fwd", "splash_pointwise_fwd"])
def test_forward_validation_errors(fn):
    lib = bd.load_library()
    d, keep = _desc()
    inf = _info()
    E = bd
    # unsupported dtype pair and head_dim
    assert _fwd(lib, fn, in_dt=0, out_dt=1, desc=d, info=inf) == E.SPLASH_ERR_UNSUPPORTED
    assert _fwd(lib, fn, D=96, desc=d, info=inf) == E.SPLASH_ERR_UNSUPPORTED
    assert b"head_dim" in lib.splash_last_error()
    assert _fwd(lib, fn, D=0, desc=d, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT
    # null mask / info / tensors
    assert _fwd(lib, fn, desc=None, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT
    assert _fwd(lib, fn, desc=d, info=None) == E.SPLASH_ERR_INVALID_ARGUMENT
    assert _fwd(lib, fn, q=None, desc=d, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT
    # misaligned pointer and stride
    assert _fwd(lib, fn, k=0x200002, desc=d, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT
    bad = [bd._I64x3(256 * 128, 256 * 128, 130)] * 4
    assert _fwd(lib, fn, strides=bad, desc=d, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT
    # rows 64 MiB or more apart (tile copies use 32-bit buffer offsets)
    far = [bd._I64x3(256 * 128, 256 * 128, 128)] * 3 + [bd._I64x3(0, 0, 1 << 25)]
    assert _fwd(lib, fn, strides=far, desc=d, info=inf) == E.SPLASH_ERR_UNSUPPORTED
    assert b"apart" in lib.splash_last_error()
    # segment ids: both or neither
    d1, keep1 = _desc(qseg=0x5000)
    assert _fwd(lib, fn, desc=d1, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT
    assert b"both or neither" in lib.splash_last_error()
    # num_mask_heads neither 1 nor H
    d2, keep2 = _desc(heads=[(1, -1, -1)] * 2)
    assert _fwd(lib, fn, H=3, desc=d2, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT
    # bad head mask fields
    d3, keep3 = _desc(heads=[(2, -1, -1)])
    assert _fwd(lib, fn, desc=d3, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT
    # metadata for another call
    assert _fwd(lib, fn, desc=d, info=_info(nq=2)) == E.SPLASH_ERR_METADATA_MISMATCH
    assert _fwd(lib, fn, desc=d, info=_info(Hm=2)) == E.SPLASH_ERR_METADATA_MISMATCH
    d4, keep4 = _desc(qseg=0x5000, kvseg=0x6000)
    assert _fwd(lib, fn, B=2, desc=d4, info=inf) == E.SPLASH_ERR_METADATA_MISMATCH  # built without segments
    # block sizes without a kernel
    assert _fwd(lib, fn, desc=d, info=_info(nq=8, nk=8, bq=32, bkv=32)) == E.SPLASH_ERR_UNSUPPORTED
    # non-finite scale
    assert _fwd(lib, fn, scale=float("nan"), desc=d, info=inf) == E.SPLASH_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("fn", ["splash_gqa_fwd", "splash_gqa_pointwise_fwd"])
def test_gqa_forward_validation_errors(fn):
    """kv_heads must divide H; the rest is checked as for splash_fwd. Every
    call here fails on the host, so nothing is launched."""
    lib = bd.load_library()
    d, keep = _desc()
    inf = _info()

    def call(H=4, kv_heads=2, desc=d, info=inf, D=128):
        st = [bd._I64x3(H * 256 * D, 256 * D, D) for _ in range(4)]
        return getattr(lib, fn)(1, 1, 1, H, kv_heads, 256, 256, D, 0x100000, st[0], 0x200000, st[1],
                                0x300000, st[2], 0x400000, st[3], 0.1, ctypes.byref(desc) if desc else None,
                                ctypes.byref(info) if info else None, None)

    assert call(kv_heads=3) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert b"kv_heads" in lib.splash_last_error()
    assert call(kv_heads=0) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(kv_heads=8) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(D=96) == bd.SPLASH_ERR_UNSUPPORTED
    assert call(info=_info(nq=2)) == bd.SPLASH_ERR_METADATA_MISMATCH


def test_mask_info_build_validation_errors():
    lib = bd.load_library()
    d, keep = _desc()
    inf = _info()

    def call(B=1, H=1, Sq=256, Skv=256, bq=64, bkv=64, desc=d, info=inf):
        return lib.splash_mask_info_build(B, H, Sq, Skv, bq, bkv, None if desc is None else ctypes.byref(desc),
                                          None if info is None else ctypes.byref(info), None)

    assert call(desc=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(info=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(bq=0) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(bq=2048) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(Sq=-5) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(info=_info(nq=3)) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(info=_info(bm=None)) == bd.SPLASH_ERR_INVALID_ARGUMENT
    d1, keep1 = _desc(kvseg=0x5000)
    assert call(desc=d1) == bd.SPLASH_ERR_INVALID_ARGUMENT
    # empty metadata: nothing to build, nothing launched
    assert call(Sq=0, info=_info(nq=0)) == bd.SPLASH_OK


def test_binding_refuses_missing_library(tmp_path):
    saved = bd._lib
    bd._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            bd.load_library(str(tmp_path / "libsplash.so"))
    finally:
        bd._lib = saved


def test_pointwise_bwd_validation_errors():
    """Host-side checks of the backward: every call here fails before any
    launch (fake device addresses are never touched)."""
    lib = bd.load_library()
    d, keep = _desc()
    row = _info(bq=64, bkv=64)
    col = _info(bq=64, bkv=64)

    def call(in_dt=1, out_dt=1, H=4, kv_heads=2, D=128, info=row, info_dkv=col, desc=d, scale=0.1, align=0):
        st = [bd._I64x3(H * 256 * D, 256 * D, D) for _ in range(7)]
        ptrs = [0x100000 * (n + 1) + align for n in range(7)]
        args = []
        for p, s in zip(ptrs, st):
            args += [p, s]
        return lib.splash_pointwise_bwd(in_dt, out_dt, 1, H, kv_heads, 256, 256, D, *args, scale,
                                        ctypes.byref(desc) if desc else None,
                                        ctypes.byref(info) if info else None,
                                        ctypes.byref(info_dkv) if info_dkv else None, None)

    assert call(kv_heads=3) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(D=96) == bd.SPLASH_ERR_UNSUPPORTED
    assert call(in_dt=0, out_dt=1) == bd.SPLASH_ERR_UNSUPPORTED
    assert call(scale=float("nan")) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(info=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(info_dkv=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert b"info_dkv" in lib.splash_last_error()
    assert call(desc=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert call(info=_info(nq=3)) == bd.SPLASH_ERR_METADATA_MISMATCH
    assert call(info_dkv=_info(nk=3)) == bd.SPLASH_ERR_METADATA_MISMATCH
    # block sizes without a compiled kernel
    assert call(info=_info(nq=8, bq=32)) == bd.SPLASH_ERR_UNSUPPORTED
    assert call(info_dkv=_info(nq=16, nk=16, bq=16, bkv=16)) == bd.SPLASH_ERR_UNSUPPORTED
    assert call(info_dkv=_info(nk=8, bkv=32)) == bd.SPLASH_ERR_UNSUPPORTED
    assert call(align=8) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert b"aligned" in lib.splash_last_error()


def test_mask_info_build_dkv_validation_errors():
    lib = bd.load_library()
    d, keep = _desc()
    assert lib.splash_mask_info_build_dkv(1, 1, 256, 256, 64, 64, ctypes.byref(d), None, None) == \
        bd.SPLASH_ERR_INVALID_ARGUMENT
    assert lib.splash_mask_info_build_dkv(1, 1, 256, 256, 64, 64, ctypes.byref(d), ctypes.byref(_info(nq=3)),
                                          None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert lib.splash_mask_info_build_dkv(1, 1, 0, 256, 64, 64, ctypes.byref(d), ctypes.byref(_info(nq=0)),
                                          None) == bd.SPLASH_OK


def test_mask_info_build_too_large_for_one_launch():
    """Metadata whose build would need more workgroups than one launch takes
    is refused on the host: columns of the dK/dV layout, and the segment-id
    classification (one wavefront per 64 entries)."""
    lib = bd.load_library()
    heads = [(1, -1, -1)] * 256
    d, keep = _desc(heads=heads)
    big = 1 << 30
    info = _info(Hm=256, nq=1, nk=big, bq=64, bkv=1)
    assert lib.splash_mask_info_build_dkv(1, 256, 64, big, 64, 1, ctypes.byref(d), ctypes.byref(info), None) == \
        bd.SPLASH_ERR_UNSUPPORTED
    ds, keep_s = _desc(qseg=0x1000, kvseg=0x2000)
    info = _info(nq=big, nk=big, bq=1, bkv=1)
    assert lib.splash_mask_info_build(1, 1, big, big, 1, 1, ctypes.byref(ds), ctypes.byref(info), None) == \
        bd.SPLASH_ERR_UNSUPPORTED
    assert b"too many metadata entries" in lib.splash_last_error()


def test_softmax_entry_points_validation_errors():
    """splash_fwd_lse, splash_softmax_bwd_preprocess and splash_softmax_bwd
    reject bad arguments on the host (nothing is launched)."""
    lib = bd.load_library()
    d, keep = _desc()
    row = _info(bq=64, bkv=64)
    st = [bd._I64x3(4 * 256 * 128, 256 * 128, 128) for _ in range(8)]
    ss = (ctypes.c_int64 * 2)(4 * 256, 256)

    def fwd_lse(lse=0x900000, strides=ss, H=4, kv_heads=2):
        return lib.splash_fwd_lse(1, 1, 1, H, kv_heads, 256, 256, 128, 0x100000, st[0], 0x200000, st[1],
                                  0x300000, st[2], 0x400000, st[3], lse, strides, 0.1, ctypes.byref(d),
                                  ctypes.byref(row), None)

    assert fwd_lse(strides=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert fwd_lse(lse=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert fwd_lse(kv_heads=3) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert fwd_lse(strides=(ctypes.c_int64 * 2)(-1, 0)) == bd.SPLASH_ERR_INVALID_ARGUMENT

    def pre(dtype=1, D=128, delta=0x900000, strides=ss):
        return lib.splash_softmax_bwd_preprocess(dtype, 1, 4, 256, D, 0x100000, st[0], 0x200000, st[1], delta,
                                                 strides, None)

    assert pre(D=96) == bd.SPLASH_ERR_UNSUPPORTED
    assert pre(dtype=7) == bd.SPLASH_ERR_UNSUPPORTED
    assert pre(delta=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert pre(strides=None) == bd.SPLASH_ERR_INVALID_ARGUMENT

    def bwd(lse=0x900000, delta=0xA00000, strides=ss, info_dkv=row):
        return lib.splash_softmax_bwd(1, 1, 1, 4, 2, 256, 256, 128, 0x100000, st[0], 0x200000, st[1], 0x300000,
                                      st[2], 0x400000, st[3], lse, delta, strides, 0x500000, st[4], 0x600000, st[5],
                                      0x700000, st[6], 0.1, ctypes.byref(d), ctypes.byref(row),
                                      ctypes.byref(info_dkv) if info_dkv else None, None)

    assert bwd(strides=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert bwd(lse=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert bwd(delta=0xA00002) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert bwd(info_dkv=None) == bd.SPLASH_ERR_INVALID_ARGUMENT


def test_misaligned_metadata_and_statistics_are_refused():
    """block_mask and data_next are read as aligned 32-bit words, and so are
    segment ids, dense-mask arrays and the log-sum-exp rows: a pointer that is
    not 4-byte aligned is refused on the host before anything is launched."""
    lib = bd.load_library()
    E = bd
    d, keep = _desc()
    assert _fwd(lib, desc=d, info=_info(bm=0x10001)) == E.SPLASH_ERR_INVALID_ARGUMENT
    assert b"aligned" in lib.splash_last_error()
    assert _fwd(lib, desc=d, info=_info(dn=0x20002)) == E.SPLASH_ERR_INVALID_ARGUMENT
    # the same through the metadata builds
    for fn in (lib.splash_mask_info_build, lib.splash_mask_info_build_dkv):
        assert fn(1, 1, 256, 256, 64, 64, ctypes.byref(d), ctypes.byref(_info(bm=0x10003)), None) == \
            E.SPLASH_ERR_INVALID_ARGUMENT
    # segment ids
    ds, keep_s = _desc(qseg=0x5002, kvseg=0x6000)
    assert _fwd(lib, desc=ds, info=_info()) == E.SPLASH_ERR_INVALID_ARGUMENT
    assert b"segment ids must be 4-byte aligned" in lib.splash_last_error()
    # the backward's two metadata structs
    st = [bd._I64x3(4 * 256 * 128, 256 * 128, 128) for _ in range(7)]
    args = []
    for n, s in enumerate(st):
        args += [0x100000 * (n + 1), s]
    for row, col in ((_info(bm=0x10001), _info()), (_info(), _info(dn=0x20001))):
        assert lib.splash_pointwise_bwd(1, 1, 1, 4, 2, 256, 256, 128, *args, 0.1, ctypes.byref(d),
                                        ctypes.byref(row), ctypes.byref(col), None) == E.SPLASH_ERR_INVALID_ARGUMENT
    # log-sum-exp output of the forward
    ss = (ctypes.c_int64 * 2)(4 * 256, 256)
    assert lib.splash_fwd_lse(1, 1, 1, 4, 2, 256, 256, 128, 0x100000, st[0], 0x200000, st[1], 0x300000, st[2],
                              0x400000, st[3], 0x900002, ss, 0.1, ctypes.byref(d), ctypes.byref(_info()),
                              None) == E.SPLASH_ERR_INVALID_ARGUMENT
    assert b"lse" in lib.splash_last_error()
    # dense-mask arrays
    for mn, mb in ((0x30002, 0x40000), (0x30000, 0x40001)):
        part = bd.PartialMasksC(mn, mb, 3)
        stf = [bd._I64x3(256 * 128, 256 * 128, 128) for _ in range(4)]
        assert lib.splash_masked_fwd(0, 1, 1, 1, 1, 1, 256, 256, 128, 0x100000, stf[0], 0x200000, stf[1],
                                     0x300000, stf[2], 0x400000, stf[3], 0.1, ctypes.byref(d),
                                     ctypes.byref(_info()), ctypes.byref(part), None) == E.SPLASH_ERR_INVALID_ARGUMENT
        assert b"dense mask arrays must be 4-byte aligned" in lib.splash_last_error()


def test_masked_bwd_and_masked_fwd_lse_validation_errors():
    """splash_masked_bwd takes the dense structs of both walks or neither;
    its flag is 0 or 1; dense arrays must be non-null and aligned;
    splash_masked_fwd_lse needs lse strides. Every call fails on the host."""
    lib = bd.load_library()
    d, keep = _desc()
    row = _info(bq=64, bkv=64)
    st = [bd._I64x3(4 * 256 * 128, 256 * 128, 128) for _ in range(7)]
    ss = (ctypes.c_int64 * 2)(4 * 256, 256)
    good = bd.PartialMasksC(0x30000, 0x40000, 2)

    def bwd(softmax=0, p1=good, p2=good, info=row, info_dkv=row):
        args = []
        for n, s in enumerate(st):
            args.append(0x100000 * (n + 1))
            args.append(s)
        return lib.splash_masked_bwd(softmax, 1, 1, 1, 4, 2, 256, 256, 128, *args[:8], 0x900000, 0xA00000, ss,
                                     *args[8:], 0.1, ctypes.byref(d), ctypes.byref(info),
                                     ctypes.byref(p1) if p1 is not None else None, ctypes.byref(info_dkv),
                                     ctypes.byref(p2) if p2 is not None else None, None)

    assert bwd(softmax=2) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert bwd(p2=None) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert b"both or neither" in lib.splash_last_error()
    assert bwd(p1=bd.PartialMasksC(None, 0x40000, 2)) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert bwd(p2=bd.PartialMasksC(0x30002, 0x40000, 2)) == bd.SPLASH_ERR_INVALID_ARGUMENT
    assert b"aligned" in lib.splash_last_error()
    assert bwd(p1=bd.PartialMasksC(0x30000, 0x40000, -1)) == bd.SPLASH_ERR_INVALID_ARGUMENT
    # dense metadata heads must agree between the walks
    assert bwd(info_dkv=_info(Hm=4, bq=64, bkv=64)) == bd.SPLASH_ERR_METADATA_MISMATCH
    stf = [bd._I64x3(4 * 256 * 128, 256 * 128, 128) for _ in range(4)]
    assert lib.splash_masked_fwd_lse(1, 1, 1, 4, 2, 256, 256, 128, 0x100000, stf[0], 0x200000, stf[1], 0x300000,
                                     stf[2], 0x400000, stf[3], 0x900000, None, 0.1, ctypes.byref(d),
                                     ctypes.byref(row), ctypes.byref(good), None) == bd.SPLASH_ERR_INVALID_ARGUMENT
