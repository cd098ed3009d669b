"""GPU parity: the HIP kernels against the CPU oracle, byte for byte.

Bar: bit-exact for every output byte the oracle defines -- 8-bit bytes, fp16
scales, packed codes, dequantized fp16 -- and untouched bytes keep their
sentinel.  Operations: ExLlamaV2 cache page (Description / I/O Contract):
fp16_to_fp8, fp8_to_fp16, fp16_to_q_kv, q_to_fp16_kv over contiguous windows
(batch_size, offset, width) and paged caches (page_size, cache_seqlens,
block_table), wbits 4 or 6.

Workloads are the seeded synthetic ones of kv_cache_quantization_kvq_amd.synth
(fp8 [1,256,8,128]; Q4 [4,2048,8,128] window 1024+512 with outliers; Q6
[8,4096,8,128] with zero tokens; paged Q4 4096 pages x 256; paged K-Q4/V-Q6
16384 pages x 256) plus small ragged shapes and edge cases.

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import numpy as np
import pytest

import oracle
from gpu_util import (SENTINEL, byte_diff, dev, gather_rows, host, need_lib, rows_view,
                      sentinel, sentinel_np, torch)
from kv_cache_quantization_kvq_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm device"
    return need_lib()


def _log(msg):
    print(msg, flush=True)


def _cs(shape, wbits):
    return (shape[0], shape[1], shape[2], shape[3] * wbits // 8)


def _ss(shape):
    return (shape[0], shape[1], shape[2], shape[3] // 32)


# ---------------------------------------------------------------- element-level sweeps
@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_scale_rule_exhaustive(kvq, wbits):
    """Device scale rule on every finite fp16 absmax vs the oracle's fp32
    divide + fp16 rounding."""
    t = torch()
    a = np.arange(0, 0x7C00, dtype=np.uint16)
    out = t.empty(a.size, dtype=t.int16, device="cuda")
    kvq.kvq_selftest_scales(dev(a), wbits, out)
    byte_diff(host(out).view(np.uint16), oracle.scale_from_absmax(a, wbits), "scales")


def test_selftest_short_output_rejected(kvq):
    """The self-test hooks reject an output shorter than their input in the
    binding, before any launch: the output and the bytes after it keep
    their sentinel."""
    t = torch()
    a = dev(np.arange(0x3C00, 0x3C00 + 64, dtype=np.uint16))
    buf = t.full((128,), 0x5A5A, dtype=t.int16, device="cuda")
    with pytest.raises(ValueError):
        kvq.kvq_selftest_scales(a, 4, buf[:63])
    n = t.arange(64, dtype=t.int32, device="cuda")
    ibuf = t.full((128,), 0x5A5A5A5A, dtype=t.int32, device="cuda")
    with pytest.raises(ValueError):
        kvq.kvq_selftest_fastdiv(n, 7, ibuf[:63])
    t.cuda.synchronize()
    assert bool((buf == 0x5A5A).all()) and bool((ibuf == 0x5A5A5A5A).all())


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_code_rule_exhaustive(kvq, wbits):
    """Device element code on every finite fp16 x under every finite fp16
    scale >= 0 (including 0 and subnormals) vs the oracle: 63488 x 31744
    pairs, in slabs of scales.  The clamping path is checked on every pair;
    the kernels' dispatch (no clamp under normal scales) on every pair of its
    domain |x/s| < Q + 1/2, which holds for all elements of the block a
    normal scale came from."""
    from concurrent.futures import ThreadPoolExecutor
    from exact16 import f16_units
    t = torch()
    Q = (1 << (wbits - 1)) - 1
    pos = np.arange(0, 0x7C00, dtype=np.uint16)
    xs = np.concatenate([pos, pos | 0x8000])            # 63488 finite values, % 8 == 0
    X2 = 2 * f16_units(xs)
    x_dev = dev(xs)
    slab = 1024
    out = t.empty((slab, xs.size), dtype=t.uint8, device="cuda")
    pool = ThreadPoolExecutor(max_workers=8)
    for s0 in range(0, pos.size, slab):
        ss = pos[s0:s0 + slab]
        want = np.stack(list(pool.map(lambda s: oracle.quant_elems(xs, int(s), wbits), ss)))
        for force in (True, False):
            kvq.kvq_selftest_codes(x_dev, dev(ss), wbits, out[:ss.size], force_clamp=force)
            got = host(out[:ss.size])
            bad = got != want
            if not force:
                S = f16_units(ss)[:, None]
                in_domain = (S < 1024) | (np.abs(X2)[None, :] < (2 * Q + 1) * S)
                bad &= in_domain
            if bad.any():
                i, j = np.argwhere(bad)[0]
                raise AssertionError("code mismatch (force_clamp=%s): x=%#06x s=%#06x gpu=%d oracle=%d"
                                     % (force, xs[j], ss[i], got[i, j], want[i, j]))
    pool.shutdown()


def _fastdiv_divisors():
    d = set(range(1, 4097))
    for k in range(1, 31):
        d.update({(1 << k) - 1, 1 << k, (1 << k) + 1})
    d.update({(1 << 31) - 1, 256, 512, 4096 * 256, 65280, 7937})
    rng = np.random.default_rng(5150)
    d.update(int(x) for x in rng.integers(4097, 1 << 31, size=200))
    return sorted(x for x in d if 1 <= x < (1 << 31))


def test_fastdiv_divider(kvq):
    """The kernels' multiply-shift row splitter vs integer division: every
    divisor 1..4096, 2^k - 1 / 2^k / 2^k + 1 up to 2^31 - 1, the workload
    divisors and 200 random ones; numerators at every multiple's edges up to
    64 d, the top of the domain and random values below 2^31."""
    t = torch()
    rng = np.random.default_rng(5151)
    top = (1 << 31) - 1
    rand = rng.integers(0, 1 << 31, size=2048, dtype=np.int64)
    for d in _fastdiv_divisors():
        k = np.arange(0, 65, dtype=np.int64) * d
        n = np.concatenate([k - 1, k, k + 1, [top, top - 1, top - d, top - d + 1], rand])
        n = np.unique(n[(n >= 0) & (n <= top)])
        nd = t.from_numpy(n.astype(np.int32)).cuda()
        out = t.empty_like(nd)
        kvq.kvq_selftest_fastdiv(nd, d, out)
        got = host(out).astype(np.int64)
        want = n // d
        if not np.array_equal(got, want):
            i = int(np.argmax(got != want))
            raise AssertionError("fastdiv: %d // %d gave %d" % (n[i], d, got[i]))


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_dequant_exhaustive_through_kernel(kvq, wbits):
    """Every (code, scale) pair for all finite scales >= 0 through the
    production dequant kernel: block i carries scale i, codes cycle."""
    Z = 1 << (wbits - 1)
    scales = np.arange(0, 0x7C00, dtype=np.uint16)
    nblk = scales.size                                   # 31744 blocks of 32
    R = 1024
    rows = nblk * 32 // R                                # 992 rows
    shape = (1, rows, 1, R)
    for phase in range(0, 1 << wbits, 32):
        u = (np.arange(nblk * 32) + phase) % (1 << wbits)
        codes = oracle.pack_bits(u.astype(np.uint8), wbits).reshape(_cs(shape, wbits))
        sc = scales.reshape(_ss(shape)).copy()
        out = sentinel(shape, torch().float16)
        kvq.kvq_q_to_fp16_kv(dev(codes), out, dev(sc), None, None, None, 1, 0, rows,
                             wbits=wbits)
        want = sentinel_np(shape, np.float16)
        oracle.q_to_fp16_kv(codes, want, sc, None, None, None, 1, 0, rows, 0, None, None, wbits)
        byte_diff(host(out), want.view(np.uint16), "dequant phase %d" % phase)
        assert Z  # (offset-binary range covered by the cycling codes)


# ---------------------------------------------------------------- contiguous round trips
def _contig_roundtrip(kvq, k, v, batch, offset, width, wbits, stream=None, what=""):
    t = torch()
    shape = k.shape
    kd, vd = dev(k), dev(v)
    kq, vq = sentinel(_cs(shape, wbits), t.uint8), sentinel(_cs(shape, wbits), t.uint8)
    ks, vs = sentinel(_ss(shape), t.float16), sentinel(_ss(shape), t.float16)
    kvq.kvq_fp16_to_q_kv(kd, kq, ks, vd, vq, vs, batch, offset, width, wbits=wbits, stream=stream)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, batch, offset, width, wbits=wbits, stream=stream)
    if stream is not None:
        stream.synchronize()
    okq, ovq = sentinel_np(_cs(shape, wbits), np.uint8), sentinel_np(_cs(shape, wbits), np.uint8)
    oks, ovs = sentinel_np(_ss(shape), np.float16), sentinel_np(_ss(shape), np.float16)
    oracle.fp16_to_q_kv(k, okq, oks, v, ovq, ovs, batch, offset, width, 0, None, None, wbits)
    oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    oracle.q_to_fp16_kv(okq, oko, oks, ovq, ovo, ovs, batch, offset, width, 0, None, None, wbits)
    byte_diff(host(kq), okq, what + " K codes")
    byte_diff(host(vq), ovq, what + " V codes")
    byte_diff(host(ks), oks.view(np.uint16), what + " K scales")
    byte_diff(host(vs), ovs.view(np.uint16), what + " V scales")
    byte_diff(host(ko), oko.view(np.uint16), what + " K dequant")
    byte_diff(host(vo), ovo.view(np.uint16), what + " V dequant")


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_max_row_length(kvq, wbits):
    """The longest token row the library accepts: heads * head_dim = 2^20
    elements (1024 segments of a row per tensor)."""
    rng = np.random.default_rng(2 ** 20 + wbits)
    shape = (2, 3, 8192, 128)
    k = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
    v = (rng.standard_normal(shape, dtype=np.float32) * 100).astype(np.float16)
    _log("max row %s wbits %d" % (shape, wbits))
    _contig_roundtrip(kvq, k, v, 2, 1, 2, wbits, what="max row")


def test_max_row_length_fp8(kvq):
    t = torch()
    rng = np.random.default_rng(2 ** 20)
    shape = (2, 3, 8192, 128)
    x = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
    o8 = sentinel(shape, t.uint8)
    kvq.kvq_fp16_to_fp8(dev(x), o8, 2, 1, 2)
    ob = sentinel(shape, t.float16)
    kvq.kvq_fp8_to_fp16(o8, ob, 2, 1, 2)
    w8, wb = sentinel_np(shape, np.uint8), sentinel_np(shape, np.float16)
    oracle.fp16_to_fp8(x, w8, 2, 1, 2)
    oracle.fp8_to_fp16(w8, wb, 2, 1, 2)
    byte_diff(host(o8), w8, "max row 8-bit")
    byte_diff(host(ob), wb.view(np.uint16), "max row widen")


def test_q4_contig_workload(kvq):
    w = synth.q4_contig()
    _log("q4_contig %s offset %d width %d" % (w.shape, w.offset, w.width))
    _contig_roundtrip(kvq, w.k, w.v, w.batch_size, w.offset, w.width, 4, what="q4_contig")


def test_q8_contig_window(kvq):
    """Block Q8 (one code per byte) on the outlier workload's caches and window."""
    w = synth.q4_contig()
    _contig_roundtrip(kvq, w.k, w.v, w.batch_size, w.offset, w.width, 8, what="q8_contig")


def test_q6_contig_workload(kvq):
    w = synth.q6_contig()
    _log("q6_contig %s" % (w.shape,))
    _contig_roundtrip(kvq, w.k, w.v, w.batch_size, w.offset, w.width, 6, what="q6_contig")


@pytest.mark.parametrize("heads,head_dim", [(1, 32), (3, 32), (1, 96), (5, 32), (2, 64),
                                             (8, 128), (3, 1376), (1, 2080)])
@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_contig_ragged_shapes(kvq, heads, head_dim, wbits):
    """Rows of 32..4128 elements: partial waves, several segments per row,
    ragged batch / window."""
    rng = np.random.default_rng(heads * 1000 + head_dim + wbits)
    shape = (3, 7, heads, head_dim)
    k = (rng.standard_normal(shape) * 2).astype(np.float16)
    v = (rng.standard_normal(shape) * 0.01).astype(np.float16)
    _log("ragged %s wbits %d" % (shape, wbits))
    for batch, offset, width in ((3, 0, 7), (2, 3, 1), (1, 6, 1)):
        _contig_roundtrip(kvq, k, v, batch, offset, width, wbits, what="ragged %s" % (shape,))


ALPHABET = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0003, 0x000A, 0x03FF, 0x0400, 0x3800,
                     0xB800, 0x3C00, 0xBC00, 0x3E00, 0x4200, 0x4700, 0xC700, 0x4900, 0x5640,
                     0x3555, 0x7BFF, 0xFBFF, 0x1234, 0x2E66, 0x4B80], np.uint16)


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_edge_value_blocks(kvq, wbits):
    """Blocks drawn from zeros of both signs, subnormals, tie makers and
    +-65504, plus all-zero blocks and blocks whose scale underflows."""
    rng = np.random.default_rng(91 + wbits)
    shape = (2, 64, 2, 128)
    n = int(np.prod(shape))
    k = ALPHABET[rng.integers(0, ALPHABET.size, size=n)].reshape(shape)
    # per block, pick a small sub-alphabet so that many blocks have tiny absmax
    v = ALPHABET[rng.integers(0, 8, size=n)].reshape(shape).copy()
    v[0, :4] = 0
    v[1, 10:12] = 0x8000
    _contig_roundtrip(kvq, k.view(np.float16), v.view(np.float16), 2, 0, 64, wbits, what="edge")


def test_contig_on_side_stream(kvq):
    t = torch()
    w = synth.q4_contig()
    s = t.cuda.Stream()
    _contig_roundtrip(kvq, w.k, w.v, 2, 100, 64, 4, stream=s, what="side stream")


def test_k_only_and_v_only(kvq):
    t = torch()
    rng = np.random.default_rng(5)
    shape = (2, 16, 2, 64)
    x = (rng.standard_normal(shape)).astype(np.float16)
    for wbits in (4, 6, 8):
        codes = sentinel(_cs(shape, wbits), t.uint8)
        sc = sentinel(_ss(shape), t.float16)
        kvq.kvq_fp16_to_q_kv(None, None, None, dev(x), codes, sc, 2, 3, 5, wbits=wbits)
        oc = sentinel_np(_cs(shape, wbits), np.uint8)
        os_ = sentinel_np(_ss(shape), np.float16)
        oracle.fp16_to_q_kv(None, None, None, x, oc, os_, 2, 3, 5, 0, None, None, wbits)
        byte_diff(host(codes), oc, "V-only codes")
        byte_diff(host(sc), os_.view(np.uint16), "V-only scales")
        out = sentinel(shape, t.float16)
        kvq.kvq_q_to_fp16_kv(codes, out, sc, None, None, None, 2, 3, 5, wbits=wbits)
        oo = sentinel_np(shape, np.float16)
        oracle.q_to_fp16_kv(oc, oo, os_, None, None, None, 2, 3, 5, 0, None, None, wbits)
        byte_diff(host(out), oo.view(np.uint16), "K-only dequant")


def test_zero_width_touches_nothing(kvq):
    t = torch()
    shape = (2, 8, 1, 32)
    x = dev(np.ones(shape, np.float16))
    codes, sc = sentinel(_cs(shape, 4), t.uint8), sentinel(_ss(shape), t.float16)
    kvq.kvq_fp16_to_q_kv(x, codes, sc, None, None, None, 2, 3, 0, wbits=4)
    kvq.kvq_fp16_to_q_kv(x, codes, sc, None, None, None, 0, 3, 4, wbits=4)
    assert (host(codes) == SENTINEL).all() and (host(sc).view(np.uint8) == SENTINEL).all()


# ---------------------------------------------------------------- paged
def _paged_check(kvq, k, v, kq, ks, vq, vs, ko, vo, shape, batch, offset, width, page_size,
                 sl, bt, wbits_k, wbits_v, n_untouched=256, what=""):
    """Compare every touched row with the oracle (rows resolved by the
    oracle), and a sample of untouched rows against the sentinel."""
    rows = oracle.call_rows(shape[0], shape[1], batch, offset, width, page_size, sl, bt)
    valid = rows[rows >= 0]
    assert np.unique(valid).size == valid.size, "aliasing rows in a test table"
    for name, src, q, s, o, wb in (("K", k, kq, ks, ko, wbits_k), ("V", v, vq, vs, vo, wbits_v)):
        if src is None:
            continue
        xin = gather_rows(src, valid)
        c, sc = oracle.quant_rows(xin, wb)
        byte_diff(gather_rows(q, valid), c, what + " %s codes" % name)
        byte_diff(gather_rows(s, valid).view(np.uint16), sc, what + " %s scales" % name)
        byte_diff(gather_rows(o, valid).view(np.uint16), oracle.dequant_rows(c, sc, wb),
                  what + " %s dequant" % name)
        total = shape[0] * shape[1]
        rng = np.random.default_rng(7)
        cand = rng.integers(0, total, size=n_untouched * 2)
        cand = np.setdiff1d(cand, valid)[:n_untouched]
        if cand.size:
            assert (gather_rows(q, cand) == SENTINEL).all(), what + " untouched codes"
            assert (gather_rows(s, cand).view(np.uint8) == SENTINEL).all(), what + " untouched scales"
            assert (gather_rows(o, cand).view(np.uint8) == SENTINEL).all(), what + " untouched dequant"
    return valid.size


def _paged_roundtrip_small(kvq, shape, batch, offset, width, sl, bt, wbits, seed):
    t = torch()
    rng = np.random.default_rng(seed)
    k = dev((rng.standard_normal(shape) * 3).astype(np.float16))
    v = dev((rng.standard_normal(shape) * 0.1).astype(np.float16))
    kq, vq = sentinel(_cs(shape, wbits), t.uint8), sentinel(_cs(shape, wbits), t.uint8)
    ks, vs = sentinel(_ss(shape), t.float16), sentinel(_ss(shape), t.float16)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    sld, btd = dev(sl), dev(bt)
    ps = shape[1]
    kvq.kvq_fp16_to_q_kv(k, kq, ks, v, vq, vs, batch, offset, width, ps, sld, btd, wbits)
    kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, batch, offset, width, ps, sld, btd, wbits)
    return _paged_check(kvq, k, v, kq, ks, vq, vs, ko, vo, shape, batch, offset, width, ps,
                        sl, bt, wbits, wbits, what="paged ps=%d" % ps)


@pytest.mark.parametrize("page_size", [1, 3, 16])
@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_paged_small_with_invalid_entries(kvq, page_size, wbits):
    """Tiny pages, tables with -1 / out-of-range pages, negative and
    past-the-table positions: those rows are skipped on both sides."""
    rng = np.random.default_rng(page_size * 10 + wbits)
    num_pages, cols, batch = 64, 6, 5
    shape = (num_pages, page_size, 2, 64)
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = perm[:batch * cols].reshape(batch, cols).copy()
    bt[0, 1] = -1
    bt[1, 2] = num_pages + 3
    sl = rng.integers(0, cols * page_size, size=batch).astype(np.int32)
    sl[2] = -2
    width = page_size * 2 + 1
    n = _paged_roundtrip_small(kvq, shape, batch, 1, width, sl, bt, wbits, seed=page_size)
    assert n > 0


def test_q4_paged_workload(kvq):
    """4096 pages x 256 tokens, batch 32, block_table [32,32] from a seeded
    permutation, cache_seqlens in [0, 7936], width 256: quantize then
    dequantize; every touched row checked, untouched rows sampled."""
    t = torch()
    w = synth.q4_paged()
    shape = w.shape
    _log("q4_paged %s" % (shape,))
    k = synth.device_normal_f16(t, shape, w.extra["device_seed"])
    v = synth.device_normal_f16(t, shape, w.extra["device_seed"] + 1)
    kq, vq = sentinel(_cs(shape, 4), t.uint8), sentinel(_cs(shape, 4), t.uint8)
    ks, vs = sentinel(_ss(shape), t.float16), sentinel(_ss(shape), t.float16)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    sl, bt = dev(w.cache_seqlens), dev(w.block_table)
    kvq.kvq_fp16_to_q_kv(k, kq, ks, v, vq, vs, w.batch_size, w.offset, w.width, w.page_size,
                         sl, bt, 4)
    kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, w.batch_size, w.offset, w.width, w.page_size,
                         sl, bt, 4)
    n = _paged_check(kvq, k, v, kq, ks, vq, vs, ko, vo, shape, w.batch_size, w.offset, w.width,
                     w.page_size, w.cache_seqlens, w.block_table, 4, 4, what="q4_paged")
    assert n == w.batch_size * w.width


def test_mix_paged_workload(kvq):
    """16384 pages x 256 tokens (8 GiB per fp16 cache), batch 64, seq up to
    65536, K at 4 bits and V at 6 bits (one call per half), plus count_match
    on 65536 int32 token ids with a planted first mismatch."""
    t = torch()
    w = synth.mix_paged()
    shape = w.shape
    _log("mix_paged %s" % (shape,))
    k = synth.device_normal_f16(t, shape, w.extra["device_seed"])
    v = synth.device_normal_f16(t, shape, w.extra["device_seed"] + 1)
    kq, vq = sentinel(_cs(shape, 4), t.uint8), sentinel(_cs(shape, 6), t.uint8)
    ks, vs = sentinel(_ss(shape), t.float16), sentinel(_ss(shape), t.float16)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    sl, bt = dev(w.cache_seqlens), dev(w.block_table)
    args = (w.batch_size, w.offset, w.width, w.page_size, sl, bt)
    kvq.kvq_fp16_to_q_kv(k, kq, ks, None, None, None, *args, 4)
    kvq.kvq_fp16_to_q_kv(None, None, None, v, vq, vs, *args, 6)
    kvq.kvq_q_to_fp16_kv(kq, ko, ks, None, None, None, *args, 4)
    kvq.kvq_q_to_fp16_kv(None, None, None, vq, vo, vs, *args, 6)
    n = _paged_check(kvq, k, v, kq, ks, vq, vs, ko, vo, shape, w.batch_size, w.offset, w.width,
                     w.page_size, w.cache_seqlens, w.block_table, 4, 6, what="mix_paged")
    assert n == w.batch_size * w.width
    a, b, m = w.extra["ids_a"], w.extra["ids_b"], w.extra["match"]
    assert kvq.kvq_count_match(a, b, a.size) == oracle.count_match(a, b, a.size) == m


# ---------------------------------------------------------------- 8-bit
def _fp8_roundtrip(kvq, x, batch, offset, width, what):
    t = torch()
    shape = x.shape
    out8 = sentinel(shape, t.uint8)
    kvq.kvq_fp16_to_fp8(dev(x), out8, batch, offset, width)
    back = sentinel(shape, t.float16)
    kvq.kvq_fp8_to_fp16(out8, back, batch, offset, width)
    o8 = sentinel_np(shape, np.uint8)
    oracle.fp16_to_fp8(x, o8, batch, offset, width)
    ob = sentinel_np(shape, np.float16)
    oracle.fp8_to_fp16(o8, ob, batch, offset, width)
    byte_diff(host(out8), o8, what + " fp8")
    byte_diff(host(back), ob.view(np.uint16), what + " fp16")


def test_fp8_contig_workload(kvq):
    w = synth.fp8_contig()
    _fp8_roundtrip(kvq, w.k, w.batch_size, w.offset, w.width, "fp8 K")
    _fp8_roundtrip(kvq, w.v, w.batch_size, w.offset, w.width, "fp8 V")


def test_fp8_all_bit_patterns(kvq):
    x = np.arange(65536, dtype=np.uint16).reshape(1, 64, 1, 1024).view(np.float16)
    _fp8_roundtrip(kvq, x, 1, 0, 64, "all fp16 patterns")
    b = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(1, 1, 1, 1024)
    t = torch()
    out = sentinel(b.shape, t.float16)
    kvq.kvq_fp8_to_fp16(dev(b), out, 1, 0, 1)
    want = sentinel_np(b.shape, np.float16)
    oracle.fp8_to_fp16(b, want, 1, 0, 1)
    byte_diff(host(out), want.view(np.uint16), "all byte patterns")


@pytest.mark.parametrize("heads,head_dim", [(1, 8), (3, 8), (5, 200), (8, 128), (2, 4104)])
def test_fp8_ragged(kvq, heads, head_dim):
    rng = np.random.default_rng(heads + head_dim)
    shape = (4, 9, heads, head_dim)
    x = rng.standard_normal(shape).astype(np.float16)
    for batch, offset, width in ((4, 0, 9), (3, 2, 5), (1, 8, 1)):
        _fp8_roundtrip(kvq, x, batch, offset, width, "fp8 %s" % (shape,))


# ---------------------------------------------------------------- graph replay
def test_graph_replay_matches_eager(kvq):
    """The paged Q4 step captured in a HIP graph: every replay (with eager
    work and synchronisation between replays) reproduces the eager bytes."""
    t = torch()
    rng = np.random.default_rng(99)
    num_pages, ps = 64, 16
    shape = (num_pages, ps, 8, 128)
    k = dev(rng.standard_normal(shape).astype(np.float16))
    v = dev(rng.standard_normal(shape).astype(np.float16))
    bt = dev(rng.permutation(num_pages).astype(np.int32)[:32].reshape(4, 8))
    sl = dev(np.array([0, 17, 60, 100], np.int32))
    outs = [t.zeros(_cs(shape, 4), dtype=t.uint8, device="cuda"),
            t.zeros(_ss(shape), dtype=t.float16, device="cuda"),
            t.zeros(_cs(shape, 4), dtype=t.uint8, device="cuda"),
            t.zeros(_ss(shape), dtype=t.float16, device="cuda"),
            t.zeros(shape, dtype=t.float16, device="cuda"),
            t.zeros(shape, dtype=t.float16, device="cuda")]
    kq, ks, vq, vs, ko, vo = outs

    def step():
        kvq.kvq_fp16_to_q_kv(k, kq, ks, v, vq, vs, 4, 0, 20, ps, sl, bt, 4)
        kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, 4, 0, 20, ps, sl, bt, 4)

    step()
    ref = [host(o).copy() for o in outs]
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        step()
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs:
            o.zero_()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for o, r in zip(outs, ref):
            byte_diff(host(o), r, "graph replay %d" % rep)


def test_paged_q4_concurrent_graph_chains(kvq):
    """The paged Q4 workload (4096 pages x 256, batch 32, width 256) in the
    benchmark's launch configuration: eight steps over four paging draws
    captured in one HIP graph as three concurrent chains (step i, draw i % 4,
    on chain i % 3, quantize then dequantize), replayed twice.  Each draw
    runs twice, on two different chains.  Every row touched by any draw is
    checked against the oracle (a row converted by several steps is
    converted from the same source, so the result does not depend on how the
    chains interleave), untouched rows are sampled against the sentinel, and
    the second replay reproduces the first byte for byte."""
    t = torch()
    w = synth.q4_paged(draws=4)
    shape = w.shape
    _log("q4_paged concurrent chains %s, %d draws" % (shape, len(w.extra["tables"])))
    k = synth.device_normal_f16(t, shape, w.extra["device_seed"])
    v = synth.device_normal_f16(t, shape, w.extra["device_seed"] + 1)
    kq, vq = sentinel(_cs(shape, 4), t.uint8), sentinel(_cs(shape, 4), t.uint8)
    ks, vs = sentinel(_ss(shape), t.float16), sentinel(_ss(shape), t.float16)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    outs = (kq, ks, vq, vs, ko, vo)
    tabs = [(dev(sl), dev(bt)) for sl, bt in w.extra["tables"]]

    def step(d):
        sl, bt = tabs[d]
        kvq.kvq_fp16_to_q_kv(k, kq, ks, v, vq, vs, w.batch_size, w.offset, w.width, w.page_size, sl, bt, 4)
        kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, w.batch_size, w.offset, w.width, w.page_size, sl, bt, 4)

    chains = [t.cuda.Stream() for _ in range(3)]
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        cap = t.cuda.current_stream()
        for c in chains:
            c.wait_stream(cap)
        for i in range(2 * len(tabs)):
            with t.cuda.stream(chains[i % 3]):
                step(i % len(tabs))
        for c in chains:
            cap.wait_stream(c)
    t.cuda.synchronize()
    g.replay()
    t.cuda.synchronize()

    touched = np.unique(np.concatenate([
        r[r >= 0] for r in (oracle.call_rows(shape[0], shape[1], w.batch_size, w.offset, w.width,
                                             w.page_size, sl, bt) for sl, bt in w.extra["tables"])]))
    for name, src, q, s, o in (("K", k, kq, ks, ko), ("V", v, vq, vs, vo)):
        c, sc = oracle.quant_rows(gather_rows(src, touched), 4)
        byte_diff(gather_rows(q, touched), c, "chains %s codes" % name)
        byte_diff(gather_rows(s, touched).view(np.uint16), sc, "chains %s scales" % name)
        byte_diff(gather_rows(o, touched).view(np.uint16), oracle.dequant_rows(c, sc, 4),
                  "chains %s dequant" % name)
        rng = np.random.default_rng(11)
        cand = np.setdiff1d(rng.integers(0, shape[0] * shape[1], size=512), touched)[:256]
        assert cand.size > 0
        assert (gather_rows(q, cand) == SENTINEL).all(), "chains %s untouched codes" % name
        assert (gather_rows(s, cand).view(np.uint8) == SENTINEL).all(), "chains %s untouched scales" % name
        assert (gather_rows(o, cand).view(np.uint8) == SENTINEL).all(), "chains %s untouched dequant" % name

    first = [o.clone() for o in outs]
    for o in outs:
        o.view(t.uint8).fill_(SENTINEL)
    t.cuda.synchronize()
    g.replay()
    t.cuda.synchronize()
    for o, f, n in zip(outs, first, ("K codes", "K scales", "V codes", "V scales", "K out", "V out")):
        assert t.equal(o.view(t.uint8), f.view(t.uint8)), "second replay differs: %s" % n


def test_concurrent_host_threads(kvq):
    """Four host threads, each with its own stream and buffers, call the
    library concurrently (20 paged Q4 round trips each, different tables per
    thread); every thread's final bytes match the oracle."""
    import threading
    t = torch()
    rng = np.random.default_rng(8080)
    num_pages, ps, B, cols = 24, 8, 3, 4
    shape = (num_pages, ps, 4, 128)
    k = rng.standard_normal(shape).astype(np.float16)
    v = (rng.standard_normal(shape) * 0.5).astype(np.float16)
    kd, vd = dev(k), dev(v)
    jobs = []
    for i in range(4):
        bt = rng.permutation(num_pages).astype(np.int32)[:B * cols].reshape(B, cols)
        sl = rng.integers(0, cols * ps - 10, size=B).astype(np.int32)
        outs = (sentinel(_cs(shape, 4), t.uint8), sentinel(_ss(shape), t.float16),
                sentinel(_cs(shape, 4), t.uint8), sentinel(_ss(shape), t.float16),
                sentinel(shape, t.float16), sentinel(shape, t.float16))
        jobs.append((sl, bt, dev(sl), dev(bt), outs, t.cuda.Stream()))
    t.cuda.synchronize()
    errors = []

    def work(job):
        try:
            sl, bt, sld, btd, (kq, ks, vq, vs, ko, vo), s = job
            with t.cuda.stream(s):
                for _ in range(20):
                    kvq.kvq_fp16_to_q_kv(kd, kq, ks, vd, vq, vs, B, 0, 10, ps, sld, btd, 4)
                    kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, B, 0, 10, ps, sld, btd, 4)
            s.synchronize()
        except Exception as e:        # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for i, (sl, bt, _, _, (kq, ks, vq, vs, ko, vo), _) in enumerate(jobs):
        okq, ovq = sentinel_np(_cs(shape, 4), np.uint8), sentinel_np(_cs(shape, 4), np.uint8)
        oks, ovs = sentinel_np(_ss(shape), np.float16), sentinel_np(_ss(shape), np.float16)
        oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
        oracle.fp16_to_q_kv(k, okq, oks, v, ovq, ovs, B, 0, 10, ps, sl, bt, 4)
        oracle.q_to_fp16_kv(okq, oko, oks, ovq, ovo, ovs, B, 0, 10, ps, sl, bt, 4)
        for got, want, n in ((kq, okq, "K codes"), (ks, oks, "K scales"), (vq, ovq, "V codes"),
                             (vs, ovs, "V scales"), (ko, oko, "K out"), (vo, ovo, "V out")):
            byte_diff(host(got), want.view(np.uint8) if want.dtype != np.uint8 else want,
                      "thread %d %s" % (i, n))


def test_fp8_batch_beyond_grid_y(kvq):
    """The contiguous 8-bit calls cap the launch's second grid dimension at
    65,535 sequences and loop over the rest: 70,000 sequences of one row
    (window offset 1, width 1 of 2 rows, 8 elements per row) against the
    oracle, untouched rows included."""
    t = torch()
    rng = np.random.default_rng(70000)
    shape = (70000, 2, 1, 8)
    x = rng.standard_normal(shape).astype(np.float16)
    o8 = sentinel(shape, t.uint8)
    ob = sentinel(shape, t.float16)
    kvq.kvq_fp16_to_fp8(dev(x), o8, 70000, 1, 1)
    kvq.kvq_fp8_to_fp16(o8, ob, 70000, 1, 1)
    w8, wb = sentinel_np(shape, np.uint8), sentinel_np(shape, np.float16)
    oracle.fp16_to_fp8(x, w8, 70000, 1, 1)
    oracle.fp8_to_fp16(w8, wb, 70000, 1, 1)
    byte_diff(host(o8), w8, "8-bit, 70,000 sequences")
    byte_diff(host(ob), wb.view(np.uint16), "fp16 back, 70,000 sequences")


# ---------------------------------------------------------------- bandwidth references
@pytest.mark.parametrize("lane_bytes,group_waves,max_waves", [(16, 1, 0), (64, 4, 0), (128, 2, 0), (32, 8, 5)])
def test_selftest_copy(kvq, lane_bytes, group_waves, max_waves):
    """The plain copy moves every byte, for sizes that end inside a tile and
    with waves striding over the tiles."""
    t = torch()
    n = 16 * (64 * 8 * 13 + 37)
    src = t.randint(0, 256, (n,), dtype=t.uint8, device="cuda")
    dst = t.zeros(n + 256, dtype=t.uint8, device="cuda")
    kvq.kvq_selftest_copy(src, dst[:n], lane_bytes, group_waves, max_waves)
    assert t.equal(dst[:n], src) and int(dst[n:].count_nonzero()) == 0


@pytest.mark.parametrize("lane_elems", [2, 4, 8])
@pytest.mark.parametrize("group_waves", [1, 4])
def test_selftest_stream(kvq, lane_elems, group_waves):
    """The uneven-traffic reference: gather writes the XOR of each lane's
    heavy-side elements, scatter writes each light element lane_elems
    times; nothing outside dst is written."""
    t = torch()
    tiles = 37
    light = 1024 * tiles
    heavy = light * lane_elems
    src = t.randint(0, 256, (heavy,), dtype=t.uint8, device="cuda")
    out = t.zeros(light + 1024, dtype=t.uint8, device="cuda")
    kvq.kvq_selftest_stream(src, out[:light], lane_elems, group_waves)
    s = host(src).view(np.uint32).reshape(tiles, lane_elems, 64, 4)
    want = np.bitwise_xor.reduce(s, axis=1).reshape(-1)
    got = host(out).view(np.uint32)
    assert np.array_equal(got[:light // 4], want) and not got[light // 4:].any()
    src2 = t.randint(0, 256, (light,), dtype=t.uint8, device="cuda")
    out2 = t.zeros(heavy + 1024, dtype=t.uint8, device="cuda")
    kvq.kvq_selftest_stream(src2, out2[:heavy], lane_elems, group_waves)
    s2 = host(src2).view(np.uint32).reshape(tiles, 1, 64, 4)
    got2 = host(out2).view(np.uint32)
    want2 = np.broadcast_to(s2, (tiles, lane_elems, 64, 4)).reshape(-1)
    assert np.array_equal(got2[:heavy // 4], want2) and not got2[heavy // 4:].any()
