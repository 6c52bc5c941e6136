"""C ABI checks that need no GPU: the library loads, exports every function tq.h declares,
its host-side codebook builder matches the oracle's tables, and argument validation
rejects bad calls before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_attention_rotate_amd as tq
from compressed_attention_rotate_amd._lib import c_cache_segment, c_format, c_tables
from oracle import tq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = tq.load()
    names = _declared()
    assert {"tq_build_codebook", "tq_quantize_kv", "tq_attend_decode", "tq_ip_search"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in tq.h but not exported"


@pytest.mark.parametrize("d", [8, 128, 256, 1024])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_host_codebook_matches_oracle_tables(d, bits):
    c, b, mse = tq.build_codebook(d, bits)
    ref = O.codebook(d, bits)
    assert np.array_equal(c.astype(np.float64), ref.centroids)
    assert np.array_equal(b.astype(np.float64), ref.bounds)
    assert abs(mse - ref.mse) < 1e-9 * ref.mse + 1e-15


def test_codebook_argument_errors():
    lib = tq.load()
    c = np.zeros(16, np.float32)
    b = np.zeros(15, np.float32)
    assert lib.tq_build_codebook(100, 2, c.ctypes.data, b.ctypes.data, None) == tq._lib.TQ_ERR_SHAPE
    assert lib.tq_build_codebook(128, 5, c.ctypes.data, b.ctypes.data, None) == tq._lib.TQ_ERR_SHAPE
    assert lib.tq_build_codebook(128, 2, None, b.ctypes.data, None) == tq._lib.TQ_ERR_ARG


def test_record_bytes_and_formats():
    assert tq.Format(128, 3, 3, 128).record_bytes() == 64          # b = 4: 4.25 bit/value with norms
    assert tq.Format(128, 2, 2, 128).record_bytes() == 48          # b = 3
    assert tq.Format(128, 3, 2, 64).record_bytes() == 56           # b = 3.5 mixed
    assert tq.Format(256, 3, 3, 256).record_bytes() == 128
    # MSE-only records drop one sign word per block
    assert tq.Format(128, 3, 3, 128, qjl=False).record_bytes() == 48
    assert tq.Format(128, 2, 2, 128, qjl=False).record_bytes() == 32
    assert tq.Format(128, 3, 2, 64, qjl=False).record_bytes() == 40
    for f in (O.Format(128, 3, 3, 128), O.Format(128, 3, 2, 64), O.Format(256, 2, 2, 256),
              O.Format(128, 3, 3, 128, False), O.Format(128, 2, 1, 96, False),
              O.Format(256, 3, 3, 256, False)):
        assert tq.Format(f.d, f.bits_lo, f.bits_hi, f.split, f.qjl).record_bytes() == f.record_bytes()
    lib = tq.load()
    for bad in ((64, 3, 3, 64), (128, 4, 4, 128), (128, 3, 2, 48), (128, 3, 2, 128), (256, 1, 1, 256)):
        for qjl in (0, 1):
            f = c_format(*bad, qjl)
            assert lib.tq_check_format(ctypes.byref(f)) == tq._lib.TQ_ERR_SHAPE
            assert lib.tq_record_bytes(ctypes.byref(f)) < 0
    f = c_format(128, 3, 3, 128, 2)                                  # qjl must be 0 or 1
    assert lib.tq_check_format(ctypes.byref(f)) == tq._lib.TQ_ERR_ARG
    assert lib.tq_record_bytes(ctypes.byref(f)) < 0


def _tables(fmt, S_ptr=0x10000):
    c, b, _ = tq.build_codebook(fmt.d, fmt.bits_lo)
    ch, bh, _ = tq.build_codebook(fmt.d, fmt.bits_hi)
    signs = np.ones(fmt.d, np.int8)
    keep = (c, b, ch, bh, signs)
    return c_tables(c.ctypes.data, b.ctypes.data, ch.ctypes.data, bh.ctypes.data, signs.ctypes.data,
                    S_ptr), keep


def test_quantize_validation_before_launch():
    lib = tq.load()
    f = c_format(128, 3, 3, 128, 1)
    t, keep = _tables(tq.Format(128, 3, 3, 128))
    fake = ctypes.c_void_p(0x20000)
    Q = lambda **kw: lib.tq_quantize_kv(ctypes.byref(kw.get("f", f)), ctypes.byref(kw.get("t", t)),
                                        kw.get("x", fake), kw.get("dt", 1), kw.get("n", 4),
                                        kw.get("d_in", 128), kw.get("ld", 128), kw.get("codes", fake),
                                        kw.get("norms", fake), None, None)
    E = tq._lib
    assert Q(n=-1) == E.TQ_ERR_ARG
    assert Q(dt=7) == E.TQ_ERR_ARG
    assert Q(d_in=129) == E.TQ_ERR_SHAPE
    assert Q(ld=100) == E.TQ_ERR_SHAPE
    assert Q(codes=ctypes.c_void_p(0x20004)) == E.TQ_ERR_ALIGN
    assert Q(x=None) == E.TQ_ERR_ARG
    assert Q(n=0) == E.TQ_OK                                          # empty is a no-op
    t2, keep2 = _tables(tq.Format(128, 3, 3, 128), S_ptr=0x10008)
    assert Q(t=t2) == E.TQ_ERR_ALIGN
    bad_signs = np.full(128, 2, np.int8)
    t3 = c_tables(t.centroids_lo, t.bounds_lo, t.centroids_hi, t.bounds_hi, bad_signs.ctypes.data, 0x10000)
    assert Q(t=t3) == E.TQ_ERR_ARG
    asym = np.array(keep[0]); asym[0] += 1e-3                         # codebook not mirror-symmetric
    t4 = c_tables(asym.ctypes.data, t.bounds_lo, t.centroids_hi, t.bounds_hi, t.signs, 0x10000)
    assert Q(t=t4) == E.TQ_ERR_ARG


def test_decode_and_search_validation_before_launch():
    lib = tq.load()
    E = tq._lib
    f = c_format(128, 3, 3, 128, 1)
    t, keep = _tables(tq.Format(128, 3, 3, 128))
    p = ctypes.c_void_p(0x40000)
    ws = tq.attend_workspace_bytes(1, 32, 8, 4096)
    assert ws > 0 and tq.attend_workspace_bytes(2, 32, 8, 4096) > ws

    def D(hq=32, hkv=8, ws_bytes=ws, tau=0.0, fv=f, q=p, fk=f, tv=t):
        return lib.tq_attend_decode(ctypes.byref(fk), ctypes.byref(t), ctypes.byref(fv), ctypes.byref(tv),
                                    q, 1, 1, hq, hkv, p, p, p, p, 4096, p, 0.088, tau, p, None, None,
                                    p, ws_bytes, None)
    assert D(hq=30) == E.TQ_ERR_SHAPE              # hq % hkv
    assert D(hq=24) == E.TQ_ERR_SHAPE              # group 3 unsupported
    assert D(ws_bytes=ws - 1) == E.TQ_ERR_WORKSPACE
    assert D(tau=-0.5) == E.TQ_ERR_ARG
    assert D(q=None) == E.TQ_ERR_ARG
    fv_bad = c_format(256, 3, 3, 256, 1)
    assert D(fv=fv_bad) == E.TQ_ERR_SHAPE
    assert D(fk=c_format(128, 3, 3, 128, 0)) == E.TQ_ERR_SHAPE   # keys need the QJL term
    f375 = c_format(128, 3, 2, 96, 1)                              # 3.75 bit: quantize-only
    assert D(fk=f375, fv=f375) == E.TQ_ERR_SHAPE
    f25 = c_format(128, 2, 1, 64, 1)                               # K b4 / V b2.5: supported
    t25, keep25 = _tables(tq.Format(128, 2, 1, 64))
    assert D(fv=f25, tv=t25, ws_bytes=ws - 1) == E.TQ_ERR_WORKSPACE  # (stops at the workspace check)
    assert D(fv=f25, ws_bytes=ws - 1) == E.TQ_ERR_ARG                # tables of another width
    f2 = c_format(256, 3, 3, 256, 1)
    t2, keep2 = _tables(tq.Format(256, 3, 3, 256))
    wsb = tq.search_workspace_bytes(100, 10, 10 ** 6, 256)
    assert wsb > 0

    def S(k=10, n_db=10 ** 6, d_in=200, ws_bytes=wsb, f=f2):
        return lib.tq_ip_search(ctypes.byref(f), ctypes.byref(t2), p, p, n_db, p, d_in, 100, k, p, p,
                                p, ws_bytes, None)
    assert S(k=0) == E.TQ_ERR_ARG
    assert S(k=65) == E.TQ_ERR_ARG
    assert S(n_db=5) == E.TQ_ERR_ARG
    assert S(d_in=300) == E.TQ_ERR_SHAPE
    assert S(ws_bytes=wsb - 1) == E.TQ_ERR_WORKSPACE
    assert S(f=c_format(256, 3, 3, 256, 0)) == E.TQ_ERR_SHAPE        # search scores need QJL


def test_segments_validation_before_launch():
    """tq_attend_decode_segments: every error is found on the host before any launch (the
    calls below run without a GPU)."""
    lib = tq.load()
    E = tq._lib
    f4, f3 = c_format(128, 3, 3, 128, 1), c_format(128, 2, 2, 128, 1)
    t4, keep4 = _tables(tq.Format(128, 3, 3, 128))
    t3, keep3 = _tables(tq.Format(128, 2, 2, 128))
    t3_other, keep3o = _tables(tq.Format(128, 2, 2, 128), S_ptr=0x18000)   # another S array
    p = ctypes.c_void_p(0x40000)
    caps = (ctypes.c_int64 * 2)(24576, 8192)
    ws = lib.tq_attend_segments_workspace_bytes(1, 32, 8, 2, caps, 128)
    assert ws == tq.attend_workspace_bytes(1, 32, 8, 24576) + tq.attend_workspace_bytes(1, 32, 8, 8192)
    assert lib.tq_attend_segments_workspace_bytes(1, 32, 8, 0, caps, 128) == -1
    assert lib.tq_attend_segments_workspace_bytes(1, 32, 8, 9, caps, 128) == -1

    def seg(fk, tk, fv, tv, cap):
        return c_cache_segment(ctypes.addressof(fk), ctypes.addressof(tk), ctypes.addressof(fv),
                               ctypes.addressof(tv), p, p, p, p, cap, p)

    def G(segs, n=None, ws_bytes=ws):
        arr = (c_cache_segment * len(segs))(*segs)
        return lib.tq_attend_decode_segments(arr, len(segs) if n is None else n, p, 1, 1, 32, 8,
                                             0.088, 0.0, p, None, p, ws_bytes, None)
    good = [seg(f3, t3, f3, t3, 24576), seg(f4, t4, f4, t4, 8192)]
    assert G(good, ws_bytes=ws - 1) == E.TQ_ERR_WORKSPACE       # (every other check passed)
    assert G(good, n=0) == E.TQ_ERR_ARG
    assert G(good, n=9) == E.TQ_ERR_ARG
    assert lib.tq_attend_decode_segments(None, 2, p, 1, 1, 32, 8, 0.088, 0.0, p, None, p, ws,
                                         None) == E.TQ_ERR_ARG
    # value tables of another rotation cannot be merged; key tables may differ
    assert G([seg(f3, t3, f3, t3_other, 24576), seg(f4, t4, f4, t4, 8192)]) == E.TQ_ERR_ARG
    assert G([seg(f3, t3_other, f3, t3, 24576), seg(f4, t4, f4, t4, 8192)],
             ws_bytes=ws - 1) == E.TQ_ERR_WORKSPACE
    # a segment's own format checks still apply
    assert G([seg(c_format(128, 3, 3, 128, 0), t4, f4, t4, 24576), seg(f4, t4, f4, t4, 8192)]) \
        == E.TQ_ERR_SHAPE


def test_strerror_names_every_code():
    lib = tq.load()
    seen = {lib.tq_strerror(c).decode() for c in range(0, -7, -1)}
    assert len(seen) == 7 and lib.tq_strerror(-99).decode() == "unknown status code"


def test_requantize_validation_before_launch():
    lib = tq.load()
    E = tq._lib
    fi, fo = c_format(128, 3, 3, 128, 1), c_format(128, 2, 2, 128, 1)
    ti, k1 = _tables(tq.Format(128, 3, 3, 128))
    to, k2 = _tables(tq.Format(128, 2, 2, 128))
    n = 1000
    cin, nin = 0x100000, 0x200000
    cout, nout, ws = 0x300000, 0x400000, 0x500000
    wsb = tq.requantize_workspace_bytes(n)
    assert wsb == n * 580 and tq.requantize_workspace_bytes(0) == 580

    def R(n=n, ci=cin, ni=nin, co=cout, no=nout, w=ws, wb=wsb, f_out=fo, t_out=to, f_in=fi, t_in=ti):
        P = ctypes.c_void_p
        return lib.tq_requantize(ctypes.byref(f_in), ctypes.byref(t_in), P(ci), P(ni), n,
                                 ctypes.byref(f_out), ctypes.byref(t_out), P(co), P(no), None,
                                 P(w), wb, None)
    assert R(n=0) == E.TQ_OK
    assert R(n=-1) == E.TQ_ERR_ARG
    assert R(wb=579) == E.TQ_ERR_WORKSPACE
    assert R(co=0x300004) == E.TQ_ERR_ALIGN
    assert R(co=cin + 64) == E.TQ_ERR_ARG                          # overlaps the input records
    assert R(w=nout + 16) == E.TQ_ERR_ARG                          # workspace overlaps norms
    assert R(f_in=fo, t_in=to, f_out=fi, t_out=ti, co=cin, no=nin) == E.TQ_ERR_ARG  # wider in place
    assert R(f_in=fo, t_in=to, f_out=fi, t_out=ti, n=0, co=cin, no=nin) == E.TQ_OK
    flipped = np.array(k2[4]); flipped[5] = -1
    t_flip = c_tables(to.centroids_lo, to.bounds_lo, to.centroids_hi, to.bounds_hi,
                      flipped.ctypes.data, 0x10000)
    assert R(t_out=t_flip) == E.TQ_ERR_ARG                         # another rotation
    f256 = c_format(256, 2, 2, 256, 1)
    assert R(f_out=f256) == E.TQ_ERR_SHAPE


def test_paged_validation_before_launch():
    lib = tq.load()
    E = tq._lib
    f = c_format(128, 3, 3, 128, 1)
    t, keep = _tables(tq.Format(128, 3, 3, 128))
    P = ctypes.c_void_p
    x, slots, cache, norms = P(0x100000), P(0x200000), P(0x300000), P(0x400000)

    def A(n_tokens=10, hkv=8, page=64, pages=4, sl=slots):
        return lib.tq_quantize_kv_paged(ctypes.byref(f), ctypes.byref(t), x, 1, n_tokens, hkv, 128,
                                        128, sl, page, pages, cache, norms, None, None)
    assert A(n_tokens=0) == E.TQ_OK
    assert A(page=96) == E.TQ_ERR_ARG                  # not a power of two
    assert A(page=32) == E.TQ_ERR_ARG                  # below one 64-token tile
    assert A(pages=0) == E.TQ_ERR_ARG
    assert A(hkv=0) == E.TQ_ERR_ARG
    assert A(sl=None) == E.TQ_ERR_ARG
    assert A(sl=P(0x200004)) == E.TQ_ERR_ALIGN
    bt, sl32, q, ws = P(0x500000), P(0x600000), P(0x700000), P(0x800000)
    wsb = tq.attend_workspace_bytes(1, 32, 8, 4 * 64)

    def D(page=64, pages=4, table=bt, mb=4, hq=32, wb=wsb):
        return lib.tq_attend_decode_paged(ctypes.byref(f), ctypes.byref(t), ctypes.byref(f),
                                          ctypes.byref(t), q, 1, 1, hq, 8, cache, norms, cache,
                                          norms, page, pages, table, mb, sl32, 0.088, 0.0, q, None,
                                          None, ws, wb, None)
    assert D(page=100) == E.TQ_ERR_ARG
    assert D(pages=0) == E.TQ_ERR_ARG
    assert D(table=None) == E.TQ_ERR_ARG
    assert D(mb=0) == E.TQ_ERR_ARG
    assert D(table=P(0x500002)) == E.TQ_ERR_ALIGN
    assert D(hq=30) == E.TQ_ERR_SHAPE
    assert D(wb=wsb - 1) == E.TQ_ERR_WORKSPACE
    assert tq.attend_workspace_bytes(1, 32, 8, 64 * 64) > wsb
    assert D(mb=64) == E.TQ_ERR_WORKSPACE              # the capacity grows with max_blocks


def test_segments_plan_sizes_every_split_partial():
    """Eight segments of 131072 tokens at batch 1 with one KV head: every segment keeps its
    own 256 splits (2048 partials per query head, merged by one combine) and the workspace
    holds all of them."""
    per = 256 * 4 * (2 + 2 * 128) * 4
    assert tq.attend_segments_workspace_bytes(1, 4, 1, [131072] * 8) == 8 * per
    assert tq.attend_workspace_bytes(1, 4, 1, 131072) == per
