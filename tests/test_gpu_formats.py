"""GPU parity of the per-tensor-format and full-prefix entry points against
the CPU oracle, byte for byte (include/kvq.h: kvq_fp16_to_kv,
kvq_kv_to_fp16, kvq_kv_to_fp16_prefix).

The page's K/V functions take one wbits for both tensors and its 8-bit
functions have no paging arguments (ExLlamaV2 cache page, Signature); these
entry points give each tensor its own format (8-bit high byte, Q4, Q6, Q8),
page the 8-bit format, and widen every cached position of each sequence
before attention (Usage section: conversion during the attention forward).

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import numpy as np
import pytest

import oracle
from gpu_util import SENTINEL, byte_diff, dev, gather_rows, host, need_lib, sentinel, sentinel_np, torch
from kv_cache_quantization_kvq_amd import synth

pytestmark = pytest.mark.gpu

FMTS = (0, 4, 6, 8)


@pytest.fixture(scope="module")
def kvq():
    assert torch().cuda.is_available(), "GPU tests need a ROCm device"
    return need_lib()


def _log(msg):
    print(msg, flush=True)


def _cshape(shape, fmt):
    return tuple(shape) if fmt == 0 else (shape[0], shape[1], shape[2], shape[3] * fmt // 8)


def _sshape(shape):
    return (shape[0], shape[1], shape[2], shape[3] // 32)


def _dev_bufs(shape, fmt):
    t = torch()
    return sentinel(_cshape(shape, fmt), t.uint8), (None if fmt == 0 else sentinel(_sshape(shape), t.float16))


def _np_bufs(shape, fmt):
    return sentinel_np(_cshape(shape, fmt), np.uint8), (None if fmt == 0 else sentinel_np(_sshape(shape), np.float16))


def _cmp(got, want, what):
    if want is None:
        assert got is None
        return
    byte_diff(host(got), want.view(np.uint8) if want.dtype != np.uint8 else want, what)


def _roundtrip(kvq, k, v, fmt_k, fmt_v, batch, offset, width, page_size=0, sl=None, bt=None, what=""):
    t = torch()
    shape = k.shape
    kd, vd = dev(k), dev(v)
    kc, ks = _dev_bufs(shape, fmt_k)
    vc, vs = _dev_bufs(shape, fmt_v)
    sld = dev(sl) if sl is not None else None
    btd = dev(bt) if bt is not None else None
    kvq.kvq_fp16_to_kv(kd, kc, ks, fmt_k, vd, vc, vs, fmt_v, batch, offset, width, page_size, sld, btd)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    kvq.kvq_kv_to_fp16(kc, ko, ks, fmt_k, vc, vo, vs, fmt_v, batch, offset, width, page_size, sld, btd)
    okc, oks = _np_bufs(shape, fmt_k)
    ovc, ovs = _np_bufs(shape, fmt_v)
    oracle.fp16_to_kv(k, okc, oks, fmt_k, v, ovc, ovs, fmt_v, batch, offset, width, page_size, sl, bt)
    oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    oracle.kv_to_fp16(okc, oko, oks, fmt_k, ovc, ovo, ovs, fmt_v, batch, offset, width, page_size, sl, bt)
    _cmp(kc, okc, what + " K compact")
    _cmp(vc, ovc, what + " V compact")
    _cmp(ks, oks, what + " K scales")
    _cmp(vs, ovs, what + " V scales")
    _cmp(ko, oko, what + " K fp16")
    _cmp(vo, ovo, what + " V fp16")


@pytest.mark.parametrize("fmt_k", FMTS)
@pytest.mark.parametrize("fmt_v", FMTS)
def test_all_format_pairs_paged(kvq, fmt_k, fmt_v):
    """Every (K, V) format pair in one launch each way, on pages of 3 tokens
    with an invalid table entry and a negative position."""
    rng = np.random.default_rng(100 + 10 * fmt_k + fmt_v)
    num_pages, ps, B, cols = 40, 3, 4, 6
    shape = (num_pages, ps, 4, 64)
    k = (rng.standard_normal(shape) * 2).astype(np.float16)
    v = (rng.standard_normal(shape) * 0.05).astype(np.float16)
    bt = rng.permutation(num_pages).astype(np.int32)[:B * cols].reshape(B, cols).copy()
    bt[2, 1] = num_pages + 5
    sl = np.array([0, 4, -1, 9], np.int32)
    _roundtrip(kvq, k, v, fmt_k, fmt_v, B, 1, 7, ps, sl, bt, what="pair (%d,%d)" % (fmt_k, fmt_v))


@pytest.mark.parametrize("heads,head_dim", [(3, 1376), (1, 32), (2, 64)])
@pytest.mark.parametrize("fmts", [(0, 8), (6, 4), (0, 0)])
def test_per_tensor_contig_ragged(kvq, heads, head_dim, fmts):
    rng = np.random.default_rng(heads + head_dim + 7 * fmts[0] + fmts[1])
    shape = (3, 6, heads, head_dim)
    k = (rng.standard_normal(shape)).astype(np.float16)
    v = (rng.standard_normal(shape) * 3).astype(np.float16)
    for batch, offset, width in ((3, 0, 6), (2, 4, 1)):
        _roundtrip(kvq, k, v, fmts[0], fmts[1], batch, offset, width, what="contig %s %s" % (shape, fmts))


@pytest.mark.parametrize("fmts", [(0, 6), (4, 8)])
def test_max_row_length_paged(kvq, fmts):
    """Rows of 2^20 elements through the per-tensor entry points on pages of
    two tokens (a position crossing a page boundary)."""
    rng = np.random.default_rng(2 ** 20 + 10 * fmts[0] + fmts[1])
    shape = (3, 2, 8192, 128)
    k = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
    v = (rng.standard_normal(shape, dtype=np.float32) * 0.01).astype(np.float16)
    bt = np.array([[2, 0]], np.int32)
    sl = np.array([1], np.int32)
    _log("max row paged %s %s" % (shape, fmts))
    _roundtrip(kvq, k, v, fmts[0], fmts[1], 1, 0, 2, 2, sl, bt, what="max row paged %s" % (fmts,))


def test_single_tensor_calls(kvq):
    t = torch()
    rng = np.random.default_rng(5)
    shape = (2, 8, 2, 64)
    x = rng.standard_normal(shape).astype(np.float16)
    for fmt in FMTS:
        c, sc = _dev_bufs(shape, fmt)
        kvq.kvq_fp16_to_kv(None, None, None, 4, dev(x), c, sc, fmt, 2, 1, 5)
        oc, osc = _np_bufs(shape, fmt)
        oracle.fp16_to_kv(None, None, None, 4, x, oc, osc, fmt, 2, 1, 5)
        _cmp(c, oc, "V-only compact")
        _cmp(sc, osc, "V-only scales")
        out = sentinel(shape, t.float16)
        kvq.kvq_kv_to_fp16(c, out, sc, fmt, None, None, None, 0, 2, 1, 5)
        oo = sentinel_np(shape, np.float16)
        oracle.kv_to_fp16(oc, oo, osc, fmt, None, None, None, 0, 2, 1, 5)
        _cmp(out, oo, "K-only fp16")


def _paged_rows_check(k, v, kc, ks, vc, vs, ko, vo, fk, fv, rows, what, n_untouched=256):
    valid = rows[rows >= 0]
    assert np.unique(valid).size == valid.size
    for name, src, c, sc, o, fmt in (("K", k, kc, ks, ko, fk), ("V", v, vc, vs, vo, fv)):
        xin = gather_rows(src, valid)
        if fmt == 0:
            # the oracle's 8-bit conversion of the gathered rows, both ways
            x4 = xin.reshape(1, xin.shape[0], 1, -1)
            want_c = np.empty(x4.shape, np.uint8)
            oracle.fp16_to_fp8(x4, want_c, 1, 0, xin.shape[0])
            want_o = np.empty(x4.shape, np.float16)
            oracle.fp8_to_fp16(want_c, want_o, 1, 0, xin.shape[0])
            want_c = want_c.reshape(xin.shape[0], -1)
            want_o = want_o.view(np.uint16).reshape(xin.shape[0], -1)
        else:
            want_c, want_s = oracle.quant_rows(xin, fmt)
            byte_diff(gather_rows(sc, valid).view(np.uint16), want_s, what + " %s scales" % name)
            want_o = oracle.dequant_rows(want_c, want_s, fmt)
        byte_diff(gather_rows(c, valid), want_c, what + " %s compact" % name)
        byte_diff(gather_rows(o, valid).view(np.uint16), want_o, what + " %s fp16" % name)
        total = src.shape[0] * src.shape[1]
        cand = np.setdiff1d(np.random.default_rng(3).integers(0, total, size=2 * n_untouched), valid)[:n_untouched]
        if cand.size:
            assert (gather_rows(c, cand) == SENTINEL).all(), what + " untouched compact"
            assert (gather_rows(o, cand).view(np.uint8) == SENTINEL).all(), what + " untouched fp16"
    return valid.size


def test_mix_paged_workload_one_launch(kvq):
    """16384 pages x 256 (8 GiB per fp16 cache), batch 64: K at 4 bits and V
    at 6 bits in a single launch each way."""
    t = torch()
    w = synth.mix_paged()
    shape = w.shape
    _log("mix_paged one launch %s" % (shape,))
    k = synth.device_normal_f16(t, shape, w.extra["device_seed"])
    v = synth.device_normal_f16(t, shape, w.extra["device_seed"] + 1)
    kc, ks = _dev_bufs(shape, 4)
    vc, vs = _dev_bufs(shape, 6)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    sl, bt = dev(w.cache_seqlens), dev(w.block_table)
    a = (w.batch_size, w.offset, w.width, w.page_size, sl, bt)
    kvq.kvq_fp16_to_kv(k, kc, ks, 4, v, vc, vs, 6, *a)
    kvq.kvq_kv_to_fp16(kc, ko, ks, 4, vc, vo, vs, 6, *a)
    rows = oracle.call_rows(shape[0], shape[1], w.batch_size, w.offset, w.width, w.page_size,
                            w.cache_seqlens, w.block_table)
    n = _paged_rows_check(k, v, kc, ks, vc, vs, ko, vo, 4, 6, rows, "mix one launch")
    assert n == w.batch_size * w.width


def test_paged_fp8_workload(kvq):
    """The 8-bit format on the paged workload (4096 pages x 256, batch 32)."""
    t = torch()
    w = synth.q4_paged()
    shape = w.shape
    k = synth.device_normal_f16(t, shape, w.extra["device_seed"])
    v = synth.device_normal_f16(t, shape, w.extra["device_seed"] + 1)
    kc, _ = _dev_bufs(shape, 0)
    vc, _ = _dev_bufs(shape, 0)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    sl, bt = dev(w.cache_seqlens), dev(w.block_table)
    a = (w.batch_size, w.offset, w.width, w.page_size, sl, bt)
    kvq.kvq_fp16_to_kv(k, kc, None, 0, v, vc, None, 0, *a)
    kvq.kvq_kv_to_fp16(kc, ko, None, 0, vc, vo, None, 0, *a)
    rows = oracle.call_rows(shape[0], shape[1], w.batch_size, w.offset, w.width, w.page_size,
                            w.cache_seqlens, w.block_table)
    assert _paged_rows_check(k, v, kc, None, vc, None, ko, vo, 0, 0, rows, "paged fp8") == w.batch_size * w.width


# ---------------------------------------------------------------- full prefix
@pytest.mark.parametrize("fmts", [(4, 6), (8, 0), (0, 0), (6, 8), (4, 4), (8, 8), (6, 6)])
def test_prefix_small(kvq, fmts):
    """Every cached position of every sequence, with an invalid table entry,
    a cap (max_len) below some lengths, and width new tokens."""
    t = torch()
    fk, fv = fmts
    rng = np.random.default_rng(300 + 10 * fk + fv)
    num_pages, ps, B, cols = 40, 4, 4, 6
    shape = (num_pages, ps, 2, 64)
    k = rng.standard_normal(shape).astype(np.float16)
    v = (rng.standard_normal(shape) * 4).astype(np.float16)
    bt = rng.permutation(num_pages).astype(np.int32)[:B * cols].reshape(B, cols).copy()
    bt[1, 2] = -3
    sl = np.array([0, 11, 17, 5], np.int32)
    width, max_len = 2, 18
    # compact caches of every row (contiguous call over all pages)
    okc, oks = _np_bufs(shape, fk)
    ovc, ovs = _np_bufs(shape, fv)
    oracle.fp16_to_kv(k, okc, oks, fk, v, ovc, ovs, fv, num_pages, 0, ps)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    kvq.kvq_kv_to_fp16_prefix(dev(okc), ko, None if oks is None else dev(oks), fk,
                              dev(ovc), vo, None if ovs is None else dev(ovs), fv,
                              B, width, max_len, dev(sl), dev(bt))
    oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    oracle.kv_to_fp16_prefix(okc, oko, oks, fk, ovc, ovo, ovs, fv, B, width, max_len, sl, bt)
    byte_diff(host(ko), oko.view(np.uint16), "prefix K")
    byte_diff(host(vo), ovo.view(np.uint16), "prefix V")


def test_prefix_paged_workload(kvq):
    """Full-prefix widen on the paged workload's tables (4096 pages x 256,
    batch 32, cache_seqlens in [0, 7936], 256 new tokens): every row in the
    prefix set is checked, untouched rows sampled."""
    t = torch()
    w = synth.q4_paged()
    shape = w.shape
    k = synth.device_normal_f16(t, shape, w.extra["device_seed"])
    kc, ks = _dev_bufs(shape, 4)
    # quantize every physical row with the contiguous single-width call
    kvq.kvq_fp16_to_q_kv(k, kc, ks, None, None, None, shape[0], 0, shape[1], wbits=4)
    ko = sentinel(shape, t.float16)
    max_len = w.block_table.shape[1] * w.page_size
    sl, bt = dev(w.cache_seqlens), dev(w.block_table)
    kvq.kvq_kv_to_fp16_prefix(kc, ko, ks, 4, None, None, None, 0, w.batch_size, w.width, max_len, sl, bt)
    rows = oracle.prefix_rows(shape[0], w.page_size, w.batch_size, w.width, max_len,
                              w.cache_seqlens, w.block_table)
    valid = rows[rows >= 0]
    assert valid.size == int(np.minimum(w.cache_seqlens.astype(np.int64) + w.width, max_len).sum())
    codes = gather_rows(kc, valid)
    scales = gather_rows(ks, valid).view(np.uint16)
    from concurrent.futures import ThreadPoolExecutor
    parts = np.array_split(np.arange(valid.size), 8)
    with ThreadPoolExecutor(8) as pool:
        want = np.concatenate(list(pool.map(lambda ix: oracle.dequant_rows(codes[ix], scales[ix], 4), parts)))
    byte_diff(gather_rows(ko, valid).view(np.uint16), want, "prefix workload")
    cand = np.setdiff1d(np.random.default_rng(4).integers(0, shape[0] * shape[1], size=512), valid)[:256]
    assert (gather_rows(ko, cand).view(np.uint8) == SENTINEL).all()


# ---------------------------------------------------------------- randomized sweep
def _random_case(rng):
    """One small seeded configuration: shape, mode, formats, window, tables."""
    heads, head_dim = int(rng.integers(1, 5)), 32 * int(rng.integers(1, 6))
    mode = ("contig", "paged", "prefix")[int(rng.integers(0, 3))]
    fk, fv = (int(f) for f in rng.choice(FMTS, 2))
    present = ("kv", "k", "v")[int(rng.choice(3, p=[0.8, 0.1, 0.1]))] if mode != "prefix" else "kv"
    c = {"mode": mode, "fk": fk, "fv": fv, "present": present}
    if mode == "contig":
        dim0, dim1 = int(rng.integers(1, 6)), int(rng.integers(1, 12))
        c["batch"] = int(rng.integers(0, dim0 + 1))
        c["offset"] = int(rng.integers(0, dim1 + 1))
        c["width"] = int(rng.integers(0, dim1 - c["offset"] + 1))
        c["ps"], c["sl"], c["bt"] = 0, None, None
    else:
        ps, B, cols = int(rng.integers(1, 10)), int(rng.integers(1, 5)), int(rng.integers(1, 5))
        dim0, dim1 = B * cols + int(rng.integers(0, 6)), ps
        bt = rng.permutation(dim0).astype(np.int32)[:B * cols].reshape(B, cols).copy()
        bad = rng.random(bt.shape) < 0.1
        bt[bad] = rng.choice(np.array([-1, -7, dim0, dim0 + 3], np.int32), size=int(bad.sum()))
        c["sl"] = rng.integers(-3, cols * ps + 3, size=B).astype(np.int32)
        c["bt"], c["batch"], c["ps"] = bt, B, ps
        c["offset"] = int(rng.integers(0, 4)) if mode == "paged" else 0
        c["width"] = int(rng.integers(0, 2 * ps + 3))
        c["max_len"] = int(rng.integers(0, cols * ps + 3))
    c["shape"] = (dim0, dim1, heads, head_dim)
    mag = 10.0 ** rng.uniform(-6, 3)
    c["k"] = np.clip(rng.standard_normal(c["shape"]) * mag, -6e4, 6e4).astype(np.float16)
    c["v"] = np.clip(rng.standard_normal(c["shape"]) * mag * 0.1, -6e4, 6e4).astype(np.float16)
    return c


def test_randomized_configs(kvq):
    """2000 seeded small configurations (contiguous, paged with invalid table
    entries and out-of-range positions, full prefix; every format pair;
    single-tensor calls) against the oracle, every byte of every buffer."""
    t = torch()
    rng = np.random.default_rng(20261203)
    for case in range(2000):
        c = _random_case(rng)
        shape, fk, fv = c["shape"], c["fk"], c["fv"]
        has_k, has_v = "k" in c["present"], "v" in c["present"]
        what = "case %d %s %s fmts (%d,%d) %s" % (case, c["mode"], shape, fk, fv, c["present"])
        sld = dev(c["sl"]) if c["sl"] is not None else None
        btd = dev(c["bt"]) if c["bt"] is not None else None
        okc, oks = _np_bufs(shape, fk)
        ovc, ovs = _np_bufs(shape, fv)
        oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
        ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
        if c["mode"] == "prefix":
            # compact caches of every row, then widen each sequence's prefix
            oracle.fp16_to_kv(c["k"], okc, oks, fk, c["v"], ovc, ovs, fv, shape[0], 0, shape[1])
            kvq.kvq_kv_to_fp16_prefix(dev(okc), ko, None if oks is None else dev(oks), fk,
                                      dev(ovc), vo, None if ovs is None else dev(ovs), fv,
                                      c["batch"], c["width"], c["max_len"], sld, btd)
            oracle.kv_to_fp16_prefix(okc, oko, oks, fk, ovc, ovo, ovs, fv, c["batch"], c["width"],
                                     c["max_len"], c["sl"], c["bt"])
            byte_diff(host(ko), oko.view(np.uint16), what + " K")
            byte_diff(host(vo), ovo.view(np.uint16), what + " V")
            continue
        kc, ks = _dev_bufs(shape, fk)
        vc, vs = _dev_bufs(shape, fv)
        kd, vd = dev(c["k"]), dev(c["v"])
        a = (c["batch"], c["offset"], c["width"], c["ps"], sld, btd)
        kvq.kvq_fp16_to_kv(kd if has_k else None, kc if has_k else None, ks if has_k else None, fk,
                           vd if has_v else None, vc if has_v else None, vs if has_v else None, fv, *a)
        kvq.kvq_kv_to_fp16(kc if has_k else None, ko if has_k else None, ks if has_k else None, fk,
                           vc if has_v else None, vo if has_v else None, vs if has_v else None, fv, *a)
        oa = (c["batch"], c["offset"], c["width"], c["ps"], c["sl"], c["bt"])
        oracle.fp16_to_kv(c["k"] if has_k else None, okc if has_k else None, oks if has_k else None, fk,
                          c["v"] if has_v else None, ovc if has_v else None, ovs if has_v else None, fv, *oa)
        oracle.kv_to_fp16(okc if has_k else None, oko if has_k else None, oks if has_k else None, fk,
                          ovc if has_v else None, ovo if has_v else None, ovs if has_v else None, fv, *oa)
        # absent tensors keep their sentinels on both sides
        _cmp(kc, okc, what + " K compact")
        _cmp(vc, ovc, what + " V compact")
        _cmp(ks, oks, what + " K scales")
        _cmp(vs, ovs, what + " V scales")
        byte_diff(host(ko), oko.view(np.uint16), what + " K fp16")
        byte_diff(host(vo), ovo.view(np.uint16), what + " V fp16")


def test_randomized_single_width(kvq):
    """1000 seeded small configurations through the one-width entry points
    (kvq_fp16_to_q_kv / kvq_q_to_fp16_kv; the page's fp16_to_q_kv and
    q_to_fp16_kv): contiguous windows and paged tables with invalid entries
    and out-of-range positions, wbits 4, 6 or 8, K and V together or one of
    them, against the oracle, every byte of every buffer."""
    t = torch()
    rng = np.random.default_rng(20261204)
    case = 0
    while case < 1000:
        c = _random_case(rng)
        if c["mode"] == "prefix":
            continue
        wb = int(rng.choice([4, 6, 8]))
        shape = c["shape"]
        has_k, has_v = "k" in c["present"], "v" in c["present"]
        what = "single-width case %d %s %s Q%d %s" % (case, c["mode"], shape, wb, c["present"])
        case += 1
        kq, vq = sentinel(_cshape(shape, wb), t.uint8), sentinel(_cshape(shape, wb), t.uint8)
        ks, vs = sentinel(_sshape(shape), t.float16), sentinel(_sshape(shape), t.float16)
        ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
        okq, ovq = sentinel_np(_cshape(shape, wb), np.uint8), sentinel_np(_cshape(shape, wb), np.uint8)
        oks, ovs = sentinel_np(_sshape(shape), np.float16), sentinel_np(_sshape(shape), np.float16)
        oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
        kd, vd = dev(c["k"]), dev(c["v"])
        sld = dev(c["sl"]) if c["sl"] is not None else None
        btd = dev(c["bt"]) if c["bt"] is not None else None
        a = (c["batch"], c["offset"], c["width"], c["ps"], sld, btd)
        kt = (kd, kq, ks) if has_k else (None, None, None)
        vt = (vd, vq, vs) if has_v else (None, None, None)
        kvq.kvq_fp16_to_q_kv(*kt, *vt, *a, wbits=wb)
        kvq.kvq_q_to_fp16_kv(*((kq, ko, ks) if has_k else (None,) * 3), *((vq, vo, vs) if has_v else (None,) * 3),
                             *a, wbits=wb)
        oa = (c["batch"], c["offset"], c["width"], c["ps"], c["sl"], c["bt"], wb)
        okt = (c["k"], okq, oks) if has_k else (None, None, None)
        ovt = (c["v"], ovq, ovs) if has_v else (None, None, None)
        oracle.fp16_to_q_kv(*okt, *ovt, *oa)
        oracle.q_to_fp16_kv(*((okq, oko, oks) if has_k else (None,) * 3),
                            *((ovq, ovo, ovs) if has_v else (None,) * 3), *oa)
        byte_diff(host(kq), okq, what + " K codes")
        byte_diff(host(vq), ovq, what + " V codes")
        byte_diff(host(ks), oks.view(np.uint16), what + " K scales")
        byte_diff(host(vs), ovs.view(np.uint16), what + " V scales")
        byte_diff(host(ko), oko.view(np.uint16), what + " K fp16")
        byte_diff(host(vo), ovo.view(np.uint16), what + " V fp16")


def test_every_entry_point_under_graph_capture(kvq):
    """One call of each device entry point captured in a single HIP graph:
    8-bit both ways, Q4 both ways, per-tensor (K Q6, V 8-bit) both ways and
    the full-prefix widen.  Three replays, with the outputs refilled eagerly
    and the device synchronised between them, each reproduce the eager
    bytes."""
    t = torch()
    rng = np.random.default_rng(404)
    num_pages, ps, B, cols = 12, 8, 3, 4
    shape = (num_pages, ps, 4, 64)
    k = dev((rng.standard_normal(shape) * 2).astype(np.float16))
    v = dev((rng.standard_normal(shape) * 0.3).astype(np.float16))
    bt = dev(rng.permutation(num_pages).astype(np.int32)[:B * cols].reshape(B, cols))
    sl = dev(np.array([2, 9, 17], np.int32))
    width, max_len = 10, cols * ps
    cshape = (2, 16, 4, 64)
    x = dev(rng.standard_normal(cshape).astype(np.float16))
    outs = {
        "x8": t.empty(cshape, dtype=t.uint8, device="cuda"),
        "xb": t.empty(cshape, dtype=t.float16, device="cuda"),
        "kq": t.empty(_cshape(shape, 4), dtype=t.uint8, device="cuda"),
        "vq": t.empty(_cshape(shape, 4), dtype=t.uint8, device="cuda"),
        "ks": t.empty(_sshape(shape), dtype=t.float16, device="cuda"),
        "vs": t.empty(_sshape(shape), dtype=t.float16, device="cuda"),
        "ko": t.empty(shape, dtype=t.float16, device="cuda"),
        "vo": t.empty(shape, dtype=t.float16, device="cuda"),
        "kc": t.empty(_cshape(shape, 6), dtype=t.uint8, device="cuda"),
        "vc": t.empty(shape, dtype=t.uint8, device="cuda"),
        "kcs": t.empty(_sshape(shape), dtype=t.float16, device="cuda"),
        "kw": t.empty(shape, dtype=t.float16, device="cuda"),
        "vw": t.empty(shape, dtype=t.float16, device="cuda"),
        "kp": t.empty(shape, dtype=t.float16, device="cuda"),
        "vp": t.empty(shape, dtype=t.float16, device="cuda"),
    }
    o = outs

    def calls():
        kvq.kvq_fp16_to_fp8(x, o["x8"], 2, 3, 9)
        kvq.kvq_fp8_to_fp16(o["x8"], o["xb"], 2, 3, 9)
        kvq.kvq_fp16_to_q_kv(k, o["kq"], o["ks"], v, o["vq"], o["vs"], B, 0, width, ps, sl, bt, 4)
        kvq.kvq_q_to_fp16_kv(o["kq"], o["ko"], o["ks"], o["vq"], o["vo"], o["vs"], B, 0, width, ps, sl, bt, 4)
        kvq.kvq_fp16_to_kv(k, o["kc"], o["kcs"], 6, v, o["vc"], None, 0, B, 0, width, ps, sl, bt)
        kvq.kvq_kv_to_fp16(o["kc"], o["kw"], o["kcs"], 6, o["vc"], o["vw"], None, 0, B, 0, width, ps, sl, bt)
        kvq.kvq_kv_to_fp16_prefix(o["kq"], o["kp"], o["ks"], 4, o["vq"], o["vp"], o["vs"], 4, B, width,
                                  max_len, sl, bt)

    def refill():
        for tns in outs.values():
            tns.view(t.uint8).fill_(SENTINEL)

    refill()
    calls()
    ref = {name: host(tns).copy() for name, tns in outs.items()}
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        calls()
    for rep in range(3):
        refill()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for name, tns in outs.items():
            byte_diff(host(tns), ref[name], "graph replay %d: %s" % (rep, name))
