"""GPU parity of the launch shapes the conversions choose by size, against
the CPU oracle, byte for byte (every output byte, untouched sentinel bytes
included).

The kernels pick their work decomposition per launch: rows whose length is
a multiple of 1024 elements are quantized two row segments of one tensor
per wave through an LDS transpose (one 32-element block per lane; with K
and V at different formats each wave takes its tensor's), or -- paged Q6 /
Q8, and any block format up to 4,096 units -- one segment per wave with a
lane pair per block; other rows one segment per wave; paged launches of 8,192 to 32,768 units are widened in runs
of 2, 4 or 8 positions of K and V (8 of one tensor) per wave with workgroups
renumbered by XCD, other paged launches one position per wave; contiguous
K + V launches up to 16,384 units in runs of 2 positions (up to 8,192
units) or 8.  These cases sit on each side
of those choices, with page sizes that make a run of positions cross pages,
invalid table entries, positions before the cache and past the table, odd
window widths (the last pair of a sequence has one live unit), rows of 2048
and 3072 elements (a pair spans two rows), one tensor only, and K and V at
different formats.  Operations: ExLlamaV2 cache page, Description of
fp16_to_q_kv / q_to_fp16_kv (paged and contiguous), plus the per-tensor and
full-prefix entry points of include/kvq.h.

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import numpy as np
import pytest

import oracle
from gpu_util import byte_diff, dev, host, need_lib, sentinel, sentinel_np, torch

pytestmark = pytest.mark.gpu


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


def _data(rng, shape, scale):
    x = rng.standard_normal(shape, dtype=np.float32) * scale
    # a few all-zero blocks and tiny values (zero and subnormal scales)
    flat = x.reshape(-1, 32)
    pick = rng.random(flat.shape[0])
    flat[pick < 0.002] = 0
    flat[(pick >= 0.002) & (pick < 0.004)] *= 1e-6
    return x.astype(np.float16)


def _tables(rng, dim0, batch, cols, ps, width, bad_frac=0.05):
    bt = rng.permutation(dim0).astype(np.int32)[:batch * cols].reshape(batch, cols).copy()
    bad = rng.random(bt.shape) < bad_frac
    bt[bad] = rng.choice(np.array([-1, -9, dim0, dim0 + 7], np.int32), size=int(bad.sum()))
    sl = rng.integers(-5, cols * ps - width + 6, size=batch).astype(np.int32)
    return sl, bt


def _roundtrip(kvq, k, v, fk, fv, batch, offset, width, ps=0, sl=None, bt=None, what=""):
    """Per-tensor entry points (K at fk, V at fv; None drops a tensor) both
    ways, compared with the oracle on every byte."""
    t = torch()
    shape = (k if k is not None else v).shape
    kd = dev(k) if k is not None else None
    vd = dev(v) if v is not None else None
    def bufs(f, present):
        if not present:
            return None, None, None, None
        c = sentinel(_cshape(shape, f), t.uint8)
        s = None if f == 0 else sentinel(_sshape(shape), t.float16)
        oc = sentinel_np(_cshape(shape, f), np.uint8)
        os_ = None if f == 0 else sentinel_np(_sshape(shape), np.float16)
        return c, s, oc, os_
    kc, ks, okc, oks = bufs(fk, k is not None)
    vc, vs, ovc, ovs = bufs(fv, v is not None)
    sld, btd = (dev(sl), dev(bt)) if ps else (None, None)
    kvq.kvq_fp16_to_kv(kd, kc, ks, fk, vd, vc, vs, fv, batch, offset, width, ps, sld, btd)
    ko = sentinel(shape, t.float16) if k is not None else None
    vo = sentinel(shape, t.float16) if v is not None else None
    kvq.kvq_kv_to_fp16(kc, ko, ks, fk, vc, vo, vs, fv, batch, offset, width, ps, sld, btd)
    oracle.fp16_to_kv(k, okc, oks, fk, v, ovc, ovs, fv, batch, offset, width, ps, sl, bt)
    oko = sentinel_np(shape, np.float16) if k is not None else None
    ovo = sentinel_np(shape, np.float16) if v is not None else None
    oracle.kv_to_fp16(okc, oko, oks, fk, ovc, ovo, ovs, fv, batch, offset, width, ps, sl, bt)
    for got, want, name in ((kc, okc, "K compact"), (ks, oks, "K scales"), (ko, oko, "K fp16"),
                            (vc, ovc, "V compact"), (vs, ovs, "V scales"), (vo, ovo, "V fp16")):
        if want is None:
            assert got is None
            continue
        byte_diff(host(got), want, "%s %s" % (what, name))


@pytest.mark.parametrize("ps", [1, 3, 16])
@pytest.mark.parametrize("fmt", [4, 6, 8, 0])
def test_paged_run_size(kvq, ps, fmt):
    """16 sequences x 256 positions of K and V (8,192 units, rows of 1024):
    runs of 4 positions cross pages of 1, 3 and 16 tokens."""
    rng = np.random.default_rng(4000 + 10 * ps + fmt)
    batch, width = 16, 256
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 5
    shape = (dim0, ps, 8, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 0.3)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    _log("paged run size ps=%d fmt=%d" % (ps, fmt))
    _roundtrip(kvq, k, v, fmt, fmt, batch, 2, width, ps, sl, bt, what="paged ps=%d fmt=%d" % (ps, fmt))


def test_paged_single_width_run_size(kvq):
    """The page's single-width calls (one wbits for K and V) at the run size,
    13 sequences x 317 positions: an odd width, 8,242 units, a grid padded
    to a multiple of 8 workgroups."""
    t = torch()
    rng = np.random.default_rng(4100)
    batch, width, ps = 13, 317, 16
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 3
    shape = (dim0, ps, 8, 128)
    k, v = _data(rng, shape, 2.0), _data(rng, shape, 0.05)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    for wbits in (4, 6, 8):
        cs, ss = _cshape(shape, wbits), _sshape(shape)
        kq, vq = sentinel(cs, t.uint8), sentinel(cs, t.uint8)
        ks, vs = sentinel(ss, t.float16), sentinel(ss, t.float16)
        ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
        kvq.kvq_fp16_to_q_kv(dev(k), kq, ks, dev(v), vq, vs, batch, 0, width, ps, dev(sl), dev(bt), wbits)
        kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, batch, 0, width, ps, dev(sl), dev(bt), wbits)
        okq, ovq = sentinel_np(cs, np.uint8), sentinel_np(cs, np.uint8)
        oks, ovs = sentinel_np(ss, np.float16), sentinel_np(ss, np.float16)
        oracle.fp16_to_q_kv(k, okq, oks, v, ovq, ovs, batch, 0, width, ps, sl, bt, wbits)
        oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
        oracle.q_to_fp16_kv(okq, oko, oks, ovq, ovo, ovs, batch, 0, width, ps, sl, bt, wbits)
        for got, want, name in ((kq, okq, "K codes"), (vq, ovq, "V codes"), (ks, oks, "K scales"),
                                (vs, ovs, "V scales"), (ko, oko, "K fp16"), (vo, ovo, "V fp16")):
            byte_diff(host(got), want, "single width Q%d %s" % (wbits, name))


@pytest.mark.parametrize("heads", [16, 24])
@pytest.mark.parametrize("fmt", [4, 6, 8, 0])
def test_long_rows(kvq, heads, fmt):
    """Rows of 2048 and 3072 elements (two or three segments: a pair of
    units spans two rows when the count is odd): contiguous at a small size
    (one unit per quantize wave) and past 4,096 units (two units per wave),
    and paged at the run size."""
    rng = np.random.default_rng(4200 + heads + fmt)
    R = heads * 128
    nseg = R // 1024
    shape = (6, 48, heads, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 4.0)
    _log("long rows R=%d fmt=%d contig" % (R, fmt))
    _roundtrip(kvq, k, v, fmt, fmt, 5, 3, 37, what="contig R=%d fmt=%d" % (R, fmt))
    # contiguous past the 4,096-unit threshold of the one-unit quantize waves
    width = 4096 // (2 * nseg * 5) + 7
    assert 5 * width * 2 * nseg > 4096
    shape = (6, width + 9, heads, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 0.25)
    _log("long rows R=%d fmt=%d contig, %d units" % (R, fmt, 5 * width * 2 * nseg))
    _roundtrip(kvq, k, v, fmt, fmt, 5, 4, width, what="contig large R=%d fmt=%d" % (R, fmt))
    # paged at the run size: units = batch * width * 2 * nseg in [8192, 16384]
    batch, ps = 8, 5
    width = 8192 // (2 * nseg * batch) + 3
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 2
    pshape = (dim0, ps, heads, 128)
    k, v = _data(rng, pshape, 1.0), _data(rng, pshape, 0.5)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    _log("long rows R=%d fmt=%d paged run size" % (R, fmt))
    _roundtrip(kvq, k, v, fmt, fmt, batch, 1, width, ps, sl, bt, what="paged R=%d fmt=%d" % (R, fmt))


@pytest.mark.parametrize("fmt", [4, 6, 8])
@pytest.mark.parametrize("width", [1024, 1025])
def test_contig_one_unit_quantize_threshold(kvq, fmt, width):
    """Contiguous K + V at 4,096 units (one unit per quantize wave, lane-pair
    blocks) and just above (two units per wave)."""
    rng = np.random.default_rng(4700 + width + fmt)
    shape = (3, 1100, 8, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 2.0)
    _log("contig one-unit threshold width=%d fmt=%d" % (width, fmt))
    _roundtrip(kvq, k, v, fmt, fmt, 2, 70, width, what="contig width=%d fmt=%d" % (width, fmt))


@pytest.mark.parametrize("fmt", [4, 6, 8])
@pytest.mark.parametrize("batch", [8, 9])
def test_paged_one_unit_quantize(kvq, fmt, batch):
    """Paged K + V at 4,096 units (8 x 256 positions: one unit per quantize
    wave for every block format) and 4,608 (9 x 256: Q6 / Q8 still one unit
    per wave, Q4 two), with pages of 7 tokens, invalid entries and positions
    before the cache and past the table."""
    rng = np.random.default_rng(4800 + 10 * batch + fmt)
    width, ps = 256, 7
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 3
    shape = (dim0, ps, 8, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 0.25)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    _log("paged one-unit batch=%d fmt=%d" % (batch, fmt))
    _roundtrip(kvq, k, v, fmt, fmt, batch, 0, width, ps, sl, bt, what="paged batch=%d fmt=%d" % (batch, fmt))


@pytest.mark.parametrize("fmt", [6, 8])
@pytest.mark.parametrize("which", ["K", "V"])
def test_paged_one_unit_quantize_long_rows_one_tensor(kvq, fmt, which):
    """Paged Q6 / Q8 with rows of 3072 elements (three segments per row, one
    per wave) and one tensor only."""
    rng = np.random.default_rng(5100 + fmt + (which == "V"))
    heads, batch, width, ps = 24, 5, 61, 4
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 1
    shape = (dim0, ps, heads, 128)
    x = _data(rng, shape, 3.0)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    k, v = (x, None) if which == "K" else (None, x)
    _log("paged one-unit long rows %s fmt=%d" % (which, fmt))
    _roundtrip(kvq, k, v, fmt, fmt, batch, 1, width, ps, sl, bt, what="paged %s R=3072 fmt=%d" % (which, fmt))


MIXED = [(fk, fv) for fk in (4, 6, 8, 0) for fv in (4, 6, 8, 0) if fk != fv]


@pytest.mark.parametrize("fmts", MIXED)
def test_mixed_formats_run_size(kvq, fmts):
    """K and V at different formats in one launch at the run size: quantize
    two units of one tensor per wave in that tensor's format, widen one
    tensor per wave, 8 positions."""
    rng = np.random.default_rng(4300 + 10 * fmts[0] + fmts[1])
    batch, width, ps = 16, 300, 7
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 1
    shape = (dim0, ps, 8, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 1.0)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    _roundtrip(kvq, k, v, fmts[0], fmts[1], batch, 0, width, ps, sl, bt, what="mixed %s" % (fmts,))


@pytest.mark.parametrize("heads", [8, 16, 24])
@pytest.mark.parametrize("fmts", [(4, 6), (0, 8), (8, 4), (6, 0)])
def test_mixed_formats_contig_and_long_rows(kvq, heads, fmts):
    """K and V at different formats on contiguous windows, and paged with
    rows of 1024, 2048 and 3072 elements (a pair of units spans two rows
    when a row has an odd number of segments)."""
    rng = np.random.default_rng(4350 + heads + 10 * fmts[0] + fmts[1])
    shape = (6, 48, heads, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 3.0)
    _log("mixed %s heads=%d contig" % (fmts, heads))
    _roundtrip(kvq, k, v, fmts[0], fmts[1], 5, 3, 37, what="mixed contig %s heads=%d" % (fmts, heads))
    batch, ps, width = 6, 5, 41
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 2
    pshape = (dim0, ps, heads, 128)
    k, v = _data(rng, pshape, 0.5), _data(rng, pshape, 2.0)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    _log("mixed %s heads=%d paged" % (fmts, heads))
    _roundtrip(kvq, k, v, fmts[0], fmts[1], batch, 1, width, ps, sl, bt, what="mixed paged %s heads=%d" % (fmts, heads))


@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("fmt", [4, 0])
def test_one_tensor_run_size(kvq, which, fmt):
    """One tensor only (the other triple absent) at the run size: one tensor
    per wave, 8 positions per run."""
    rng = np.random.default_rng(4400 + fmt + (which == "v"))
    batch, width, ps = 32, 400, 32
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 4
    shape = (dim0, ps, 8, 128)
    x = _data(rng, shape, 1.0)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    k, v = (x, None) if which == "k" else (None, x)
    _roundtrip(kvq, k, v, fmt, fmt, batch, 0, width, ps, sl, bt, what="only %s fmt=%d" % (which, fmt))


def test_contig_run_size_odd(kvq):
    """Contiguous windows at the run size with an odd width: 16 x 301
    positions of K and V (9,632 units)."""
    rng = np.random.default_rng(4500)
    shape = (17, 400, 8, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 0.01)
    for fmt in (4, 6, 8, 0):
        _roundtrip(kvq, k, v, fmt, fmt, 16, 57, 301, what="contig odd fmt=%d" % fmt)


@pytest.mark.parametrize("fmts", [(4, 4), (6, 0)])
def test_prefix_run_size(kvq, fmts):
    """Full-prefix widen at the run size: 8 sequences x 1024 positions of K
    and V (16,384 units), lengths well below the cap so most runs end inside
    the cache, invalid table entries."""
    t = torch()
    fk, fv = fmts
    rng = np.random.default_rng(4600 + 10 * fk + fv)
    B, ps, cols = 8, 16, 64
    num_pages = B * cols + 9
    shape = (num_pages, ps, 8, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 2.0)
    bt = rng.permutation(num_pages).astype(np.int32)[:B * cols].reshape(B, cols).copy()
    bt[rng.random(bt.shape) < 0.03] = -2
    sl = rng.integers(-3, 990, size=B).astype(np.int32)
    width, max_len = 7, cols * ps
    okc = sentinel_np(_cshape(shape, fk), np.uint8)
    oks = None if fk == 0 else sentinel_np(_sshape(shape), np.float16)
    ovc = sentinel_np(_cshape(shape, fv), np.uint8)
    ovs = None if fv == 0 else sentinel_np(_sshape(shape), np.float16)
    oracle.fp16_to_kv(k, okc, oks, fk, v, ovc, ovs, fv, num_pages, 0, ps)
    ko, vo = sentinel(shape, t.float16), sentinel(shape, t.float16)
    _log("prefix run size %s" % (fmts,))
    kvq.kvq_kv_to_fp16_prefix(dev(okc), ko, None if oks is None else dev(oks), fk,
                              dev(ovc), vo, None if ovs is None else dev(ovs), fv,
                              B, width, max_len, dev(sl), dev(bt))
    oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    oracle.kv_to_fp16_prefix(okc, oko, oks, fk, ovc, ovo, ovs, fv, B, width, max_len, sl, bt)
    byte_diff(host(ko), oko.view(np.uint16), "prefix run size K")
    byte_diff(host(vo), ovo.view(np.uint16), "prefix run size V")


@pytest.mark.parametrize("R", [512, 768, 1024])
def test_contig_small_runs(kvq, R):
    """Contiguous K + V launches of at most 8,192 units (two positions per
    wave) with an odd width, rows of one full, one half and one guarded
    partial segment: 5 x 333 positions."""
    rng = np.random.default_rng(4700 + R)
    shape = (6, 400, R // 128, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 3.0)
    for fmt in (4, 6, 8, 0):
        _log("contig small runs R=%d fmt=%d" % (R, fmt))
        _roundtrip(kvq, k, v, fmt, fmt, 5, 41, 333, what="contig small R=%d fmt=%d" % (R, fmt))


def _absmax_blocks(rng):
    """One 32-element block per finite fp16 magnitude m (0 .. 65504): one
    element is +-m at a random position, the others random magnitudes up to
    m with random signs; then blocks of -0 only and of mixed zeros."""
    m = np.arange(0x7C00, dtype=np.uint16)
    others = (rng.random((m.size, 32)) * (m[:, None].astype(np.float64) + 1)).astype(np.uint16)
    others = np.minimum(others, m[:, None])
    pos = rng.integers(0, 32, size=m.size)
    others[np.arange(m.size), pos] = m
    sign = (rng.random(others.shape) < 0.5).astype(np.uint16) << 15
    blocks = others | sign
    neg_zero = np.full((4, 32), 0x8000, np.uint16)
    mixed_zero = ((rng.random((4, 32)) < 0.5).astype(np.uint16) << 15)
    return np.concatenate([blocks, neg_zero, mixed_zero]).view(np.float16)


@pytest.mark.parametrize("R,copies", [(1024, 1), (1024, 5), (1056, 1)])
def test_block_absmax_every_magnitude(kvq, R, copies):
    """The block maximum of |x| (scale and codes) for every finite fp16
    magnitude as the block's largest element, either sign, plus blocks of
    negative and mixed zeros, Q4 / Q6 / Q8, through each quantize kernel:
    rows of 1024 in one launch of about 1,000 units (one unit per wave,
    lane-pair blocks) and, the block set repeated 5 times, of about 5,000
    units (two units per wave, block per lane), and rows of 1056 (one unit
    per wave, guarded partial segment)."""
    rng = np.random.default_rng(4800 + R)
    blocks = np.tile(_absmax_blocks(rng), (copies, 1))
    per_row = R // 32
    rows = -(-blocks.shape[0] // per_row)
    assert (rows > 4096) == (copies > 1)   # the launch rule's threshold between the two R = 1024 kernels
    flat = np.zeros((rows * per_row, 32), np.float16)
    flat[:blocks.shape[0]] = blocks
    x = flat.reshape(1, rows, R // 32, 32)
    for fmt in (4, 6, 8):
        _log("block absmax R=%d copies=%d fmt=%d" % (R, copies, fmt))
        _roundtrip(kvq, x, None, fmt, fmt, 1, 0, rows, what="absmax R=%d x%d Q%d" % (R, copies, fmt))


@pytest.mark.parametrize("batch", [48, 70])
@pytest.mark.parametrize("fmt", [4, 6, 8, 0])
def test_paged_large_launches(kvq, batch, fmt):
    """Paged K + V launches past 16,384 units: 48 x 300 positions (28,800
    units, widened in runs of 8 positions per wave for Q4 and 8-bit, 4 for
    Q6 and Q8) and 70 x 300 (42,000 units, one position per wave), both with
    workgroups renumbered by XCD over a grid padded to a multiple of 8 (Q6
    and Q8 quantized one unit per wave); pages of 16 tokens, invalid
    entries."""
    rng = np.random.default_rng(4900 + batch + fmt)
    width, ps = 300, 16
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 3
    shape = (dim0, ps, 8, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 0.7)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    _log("paged large launch batch=%d fmt=%d" % (batch, fmt))
    _roundtrip(kvq, k, v, fmt, fmt, batch, 1, width, ps, sl, bt, what="paged large b=%d fmt=%d" % (batch, fmt))


@pytest.mark.parametrize("batch", [16, 48])
@pytest.mark.parametrize("fmt", [4, 6, 0])
@pytest.mark.parametrize("heads", [4, 6])
def test_paged_run_lengths_short_rows(kvq, heads, fmt, batch):
    """Paged K + V launches with rows of 512 elements (one chunk per lane)
    and 768 (a guarded partial segment): 16 x 260 positions (8,320 units,
    runs of 2 positions) and 48 x 260 (24,960 units: runs of 8 for Q4 and
    8-bit, 4 for Q6); pages of 16 tokens, invalid entries."""
    rng = np.random.default_rng(5000 + 100 * heads + 10 * fmt + batch)
    width, ps = 260, 16
    cols = (width + 12) // ps + 2
    dim0 = batch * cols + 3
    shape = (dim0, ps, heads, 128)
    k, v = _data(rng, shape, 1.0), _data(rng, shape, 0.5)
    sl, bt = _tables(rng, dim0, batch, cols, ps, width)
    _log("paged run lengths R=%d fmt=%d batch=%d" % (heads * 128, fmt, batch))
    _roundtrip(kvq, k, v, fmt, fmt, batch, 2, width, ps, sl, bt,
               what="paged runs R=%d fmt=%d b=%d" % (heads * 128, fmt, batch))


# ---------------------------------------------------------------- randomized run sizes
_RUN_ROWS = ((8, 128), (16, 64), (4, 256), (16, 128), (24, 128))   # R = 1024, 1024, 1024, 2048, 3072
_FMTS = (4, 6, 8, 0)


def _random_run_case(rng):
    """One seeded configuration at run sizes: rows of 1024 to 3072 elements,
    2,000 to 14,000 units (both sides of the 4,096-unit one-unit quantize
    threshold and of the 8,192-unit widen runs), contiguous or paged (page
    sizes 1 to 64, invalid table entries, positions before the cache and
    past the table), one format or two, both tensors or one."""
    heads, head_dim = _RUN_ROWS[int(rng.integers(0, len(_RUN_ROWS)))]
    nseg = heads * head_dim // 1024
    present = ("kv", "k", "v")[int(rng.choice(3, p=[0.7, 0.15, 0.15]))]
    ntens = 2 if present == "kv" else 1
    fk = int(rng.choice(_FMTS))
    fv = fk if rng.random() < 0.6 else int(rng.choice(_FMTS))
    units = int(rng.integers(2000, 14001))
    rows = max(1, units // (ntens * nseg))
    batch = int(rng.integers(1, 65))
    width = max(1, rows // batch)
    c = {"present": present, "fk": fk, "fv": fv, "batch": batch, "width": width}
    if rng.random() < 0.4:
        offset = int(rng.integers(0, 6))
        c.update(ps=0, sl=None, bt=None, offset=offset,
                 shape=(batch + int(rng.integers(0, 3)), width + offset + int(rng.integers(0, 4)), heads, head_dim))
    else:
        ps = int(rng.choice([1, 3, 16, 64]))
        cols = -(-(width + 16) // ps) + 1
        dim0 = batch * cols + int(rng.integers(0, 5))
        sl, bt = _tables(rng, dim0, batch, cols, ps, width)
        c.update(ps=ps, sl=sl, bt=bt, offset=int(rng.integers(0, 4)), shape=(dim0, ps, heads, head_dim))
    return c


def test_randomized_run_sizes(kvq):
    """40 seeded configurations at run sizes through the per-tensor entry
    points (one common format takes the same kernels as the one-width
    calls), both directions, against the oracle on every byte."""
    rng = np.random.default_rng(20261205)
    for case in range(40):
        c = _random_run_case(rng)
        k = _data(rng, c["shape"], 1.0) if "k" in c["present"] else None
        v = _data(rng, c["shape"], 0.2) if "v" in c["present"] else None
        what = "run case %d: %s %s fmts (%d,%d) batch %d width %d ps %d" % (
            case, c["present"], c["shape"], c["fk"], c["fv"], c["batch"], c["width"], c["ps"])
        _log(what)
        _roundtrip(kvq, k, v, c["fk"], c["fv"], c["batch"], c["offset"], c["width"], c["ps"], c["sl"], c["bt"],
                   what=what)
