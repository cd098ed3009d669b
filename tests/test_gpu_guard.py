"""Out-of-bounds write checks: every device buffer of a call is carved out of
a larger allocation with 256 sentinel bytes on both sides, and after the
call the guard bytes must be unchanged.  The shapes exercise the guarded
kernels (row segments shorter than a full wave, chunk tails), the 12-byte
Q6 stores and the 8-bit chunk tails, and the run kernels of rows of 1024
and 3072 elements (one- and two-unit quantize waves, runs of positions);
windows and tables reach the first and last rows of each buffer.  Outputs are also compared with the oracle.
(Operations: ExLlamaV2 cache page, Description / I/O Contract: outputs are
written in place on the touched rows only.)

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import numpy as np
import pytest

import oracle
from gpu_util import SENTINEL, byte_diff, host, need_lib, sentinel_np, torch

pytestmark = pytest.mark.gpu

GUARD = 256


@pytest.fixture(scope="module")
def kvq():
    assert torch().cuda.is_available(), "GPU tests need a ROCm device"
    return need_lib()


class Guarded:
    """A device tensor of `shape` / `dtype` inside a sentinel-filled block
    with GUARD bytes before and after it."""

    def __init__(self, shape, dtype, init=None):
        t = torch()
        n = int(np.prod(shape)) * t.empty((), dtype=dtype).element_size()
        self.block = t.full((n + 2 * GUARD,), SENTINEL, dtype=t.uint8, device="cuda")
        self.tensor = self.block[GUARD:GUARD + n].view(dtype).view(shape)
        if init is not None:
            src = t.from_numpy(np.ascontiguousarray(init).view(np.uint8).reshape(-1)).cuda()
            self.block[GUARD:GUARD + n].copy_(src)

    def check(self, what):
        b = host(self.block)
        bad = np.nonzero(np.concatenate([b[:GUARD], b[-GUARD:]]) != SENTINEL)[0]
        assert bad.size == 0, "%s: %d guard bytes written" % (what, bad.size)


def _cs(shape, fmt):
    return tuple(shape) if fmt == 0 else (shape[0], shape[1], shape[2], shape[3] * fmt // 8)


def _ss(shape):
    return (shape[0], shape[1], shape[2], shape[3] // 32)


SHAPES = [(2, 5, 3, 96), (1, 3, 5, 1376), (2, 2, 1, 32)]
# rows of 1024 and 3072 elements (the run kernels): 20 units (one unit per
# quantize wave), 4,206 units (two per wave, an odd count per sequence) and
# 8,400 units (two per wave, three segments per row)
RUN_SHAPES = [(2, 5, 8, 128), (3, 701, 8, 128), (2, 700, 24, 128)]


@pytest.mark.parametrize("shape", SHAPES)
def test_guard_fp8_contig(kvq, shape):
    t = torch()
    rng = np.random.default_rng(shape[3])
    x = rng.standard_normal(shape).astype(np.float16)
    gi = Guarded(shape, t.float16, x)
    g8 = Guarded(shape, t.uint8)
    gb = Guarded(shape, t.float16)
    batch, offset, width = shape[0], 1, shape[1] - 1            # reaches the last row
    kvq.kvq_fp16_to_fp8(gi.tensor, g8.tensor, batch, offset, width)
    kvq.kvq_fp8_to_fp16(g8.tensor, gb.tensor, batch, offset, width)
    w8, wb = sentinel_np(shape, np.uint8), sentinel_np(shape, np.float16)
    oracle.fp16_to_fp8(x, w8, batch, offset, width)
    oracle.fp8_to_fp16(w8, wb, batch, offset, width)
    byte_diff(host(g8.tensor), w8, "fp8")
    byte_diff(host(gb.tensor), wb.view(np.uint16), "fp16")
    for g, n in ((gi, "input"), (g8, "8-bit"), (gb, "fp16 out")):
        g.check("fp8 %s %s" % (shape, n))


@pytest.mark.parametrize("shape", SHAPES + RUN_SHAPES)
@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_guard_q_contig(kvq, shape, wbits):
    t = torch()
    rng = np.random.default_rng(shape[3] + wbits)
    k = rng.standard_normal(shape).astype(np.float16)
    v = (rng.standard_normal(shape) * 0.1).astype(np.float16)
    gk, gv = Guarded(shape, t.float16, k), Guarded(shape, t.float16, v)
    gkq, gvq = Guarded(_cs(shape, wbits), t.uint8), Guarded(_cs(shape, wbits), t.uint8)
    gks, gvs = Guarded(_ss(shape), t.float16), Guarded(_ss(shape), t.float16)
    gko, gvo = Guarded(shape, t.float16), Guarded(shape, t.float16)
    batch, offset, width = shape[0], 0, shape[1]                 # every row, first to last
    kvq.kvq_fp16_to_q_kv(gk.tensor, gkq.tensor, gks.tensor, gv.tensor, gvq.tensor, gvs.tensor,
                         batch, offset, width, wbits=wbits)
    kvq.kvq_q_to_fp16_kv(gkq.tensor, gko.tensor, gks.tensor, gvq.tensor, gvo.tensor, gvs.tensor,
                         batch, offset, width, wbits=wbits)
    okq, ovq = sentinel_np(_cs(shape, wbits), np.uint8), sentinel_np(_cs(shape, wbits), np.uint8)
    oks, ovs = sentinel_np(_ss(shape), np.float16), sentinel_np(_ss(shape), np.float16)
    oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    oracle.fp16_to_q_kv(k, okq, oks, v, ovq, ovs, batch, offset, width, 0, None, None, wbits)
    oracle.q_to_fp16_kv(okq, oko, oks, ovq, ovo, ovs, batch, offset, width, 0, None, None, wbits)
    byte_diff(host(gkq.tensor), okq, "K codes")
    byte_diff(host(gvq.tensor), ovq, "V codes")
    byte_diff(host(gks.tensor), oks.view(np.uint16), "K scales")
    byte_diff(host(gvs.tensor), ovs.view(np.uint16), "V scales")
    byte_diff(host(gko.tensor), oko.view(np.uint16), "K out")
    byte_diff(host(gvo.tensor), ovo.view(np.uint16), "V out")
    for g, n in ((gk, "K in"), (gv, "V in"), (gkq, "K codes"), (gvq, "V codes"), (gks, "K scales"),
                 (gvs, "V scales"), (gko, "K out"), (gvo, "V out")):
        g.check("Q%d %s %s" % (wbits, shape, n))


@pytest.mark.parametrize("fmts", [(0, 6), (4, 8), (6, 0), (8, 4)])
@pytest.mark.parametrize("head_dim", [96, 1376])
def test_guard_per_tensor_paged_and_prefix(kvq, fmts, head_dim):
    """Pages of 3 tokens; the tables hold the first and the last physical
    page: the last row (page dim0 - 1, slot 2) is converted by the window
    calls and row 0 by the prefix widen."""
    t = torch()
    fk, fv = fmts
    rng = np.random.default_rng(head_dim + 10 * fk + fv)
    num_pages, ps, B, cols = 7, 3, 2, 3
    shape = (num_pages, ps, 2, head_dim)
    k = rng.standard_normal(shape).astype(np.float16)
    v = (rng.standard_normal(shape) * 3).astype(np.float16)
    bt = np.array([[num_pages - 1, 2, 4], [0, 5, 1]], np.int32)
    sl = np.array([0, 1], np.int32)
    width = cols * ps - 1                                         # sequence 1 reaches its last slot
    gsl, gbt = Guarded(sl.shape, t.int32, sl), Guarded(bt.shape, t.int32, bt)
    gk, gv = Guarded(shape, t.float16, k), Guarded(shape, t.float16, v)
    gkc, gvc = Guarded(_cs(shape, fk), t.uint8), Guarded(_cs(shape, fv), t.uint8)
    gks = Guarded(_ss(shape), t.float16) if fk else None
    gvs = Guarded(_ss(shape), t.float16) if fv else None
    gko, gvo = Guarded(shape, t.float16), Guarded(shape, t.float16)
    gpo, gpv = Guarded(shape, t.float16), Guarded(shape, t.float16)
    ten = lambda g: None if g is None else g.tensor
    a = (B, 0, width, ps, gsl.tensor, gbt.tensor)
    kvq.kvq_fp16_to_kv(gk.tensor, gkc.tensor, ten(gks), fk, gv.tensor, gvc.tensor, ten(gvs), fv, *a)
    kvq.kvq_kv_to_fp16(gkc.tensor, gko.tensor, ten(gks), fk, gvc.tensor, gvo.tensor, ten(gvs), fv, *a)
    max_len = cols * ps
    kvq.kvq_kv_to_fp16_prefix(gkc.tensor, gpo.tensor, ten(gks), fk, gvc.tensor, gpv.tensor, ten(gvs), fv,
                              B, 2, max_len, gsl.tensor, gbt.tensor)
    okc, ovc = sentinel_np(_cs(shape, fk), np.uint8), sentinel_np(_cs(shape, fv), np.uint8)
    oks = sentinel_np(_ss(shape), np.float16) if fk else None
    ovs = sentinel_np(_ss(shape), np.float16) if fv else None
    oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    opo, opv = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    oracle.fp16_to_kv(k, okc, oks, fk, v, ovc, ovs, fv, B, 0, width, ps, sl, bt)
    oracle.kv_to_fp16(okc, oko, oks, fk, ovc, ovo, ovs, fv, B, 0, width, ps, sl, bt)
    oracle.kv_to_fp16_prefix(okc, opo, oks, fk, ovc, opv, ovs, fv, B, 2, max_len, sl, bt)
    byte_diff(host(gkc.tensor), okc, "K compact")
    byte_diff(host(gvc.tensor), ovc, "V compact")
    byte_diff(host(gko.tensor), oko.view(np.uint16), "K out")
    byte_diff(host(gvo.tensor), ovo.view(np.uint16), "V out")
    byte_diff(host(gpo.tensor), opo.view(np.uint16), "K prefix")
    byte_diff(host(gpv.tensor), opv.view(np.uint16), "V prefix")
    for g, n in ((gsl, "cache_seqlens"), (gbt, "block_table"), (gk, "K in"), (gv, "V in"), (gkc, "K compact"),
                 (gvc, "V compact"), (gks, "K scales"), (gvs, "V scales"), (gko, "K out"), (gvo, "V out"),
                 (gpo, "K prefix"), (gpv, "V prefix")):
        if g is not None:
            g.check("per-tensor %s %s %s" % (fmts, head_dim, n))


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_guard_paged_run_size(kvq, wbits):
    """9 sequences x 256 positions of K and V in pages of 16 tokens (4,608
    units: two units per Q4 quantize wave, one for Q6 / Q8; one position
    per dequantize wave), the tables holding the first and the last
    physical page: no byte outside any buffer is written."""
    t = torch()
    rng = np.random.default_rng(7700 + wbits)
    B, width, ps = 9, 256, 16
    cols = width // ps + 1
    num_pages = B * cols
    shape = (num_pages, ps, 8, 128)
    bt = rng.permutation(num_pages).astype(np.int32).reshape(B, cols)
    for want, at in ((num_pages - 1, (0, 0)), (0, (B - 1, cols - 2))):   # both live (positions < 256)
        w = np.argwhere(bt == want)[0]
        bt[tuple(w)], bt[at] = bt[at], want
    sl = np.zeros(B, np.int32)
    k = rng.standard_normal(shape).astype(np.float16)
    v = (rng.standard_normal(shape) * 0.5).astype(np.float16)
    gsl, gbt = Guarded(sl.shape, t.int32, sl), Guarded(bt.shape, t.int32, bt)
    gk, gv = Guarded(shape, t.float16, k), Guarded(shape, t.float16, v)
    gkq, gvq = Guarded(_cs(shape, wbits), t.uint8), Guarded(_cs(shape, wbits), t.uint8)
    gks, gvs = Guarded(_ss(shape), t.float16), Guarded(_ss(shape), t.float16)
    gko, gvo = Guarded(shape, t.float16), Guarded(shape, t.float16)
    a = (B, 0, width, ps, gsl.tensor, gbt.tensor)
    kvq.kvq_fp16_to_q_kv(gk.tensor, gkq.tensor, gks.tensor, gv.tensor, gvq.tensor, gvs.tensor, *a, wbits=wbits)
    kvq.kvq_q_to_fp16_kv(gkq.tensor, gko.tensor, gks.tensor, gvq.tensor, gvo.tensor, gvs.tensor, *a, wbits=wbits)
    okq, ovq = sentinel_np(_cs(shape, wbits), np.uint8), sentinel_np(_cs(shape, wbits), np.uint8)
    oks, ovs = sentinel_np(_ss(shape), np.float16), sentinel_np(_ss(shape), np.float16)
    oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    oracle.fp16_to_q_kv(k, okq, oks, v, ovq, ovs, B, 0, width, ps, sl, bt, wbits)
    oracle.q_to_fp16_kv(okq, oko, oks, ovq, ovo, ovs, B, 0, width, ps, sl, bt, wbits)
    for got, want, name in ((gkq, okq, "K codes"), (gvq, ovq, "V codes"), (gks, oks.view(np.uint16), "K scales"),
                            (gvs, ovs.view(np.uint16), "V scales"), (gko, oko.view(np.uint16), "K out"),
                            (gvo, ovo.view(np.uint16), "V out")):
        byte_diff(host(got.tensor), want, "paged run Q%d %s" % (wbits, name))
    for g, n in ((gsl, "cache_seqlens"), (gbt, "block_table"), (gk, "K in"), (gv, "V in"), (gkq, "K codes"),
                 (gvq, "V codes"), (gks, "K scales"), (gvs, "V scales"), (gko, "K out"), (gvo, "V out")):
        g.check("paged run Q%d %s" % (wbits, n))


class Offset:
    """A device tensor whose base address is `off` bytes past a 256-byte
    boundary (16-byte aligned, as the library requires, but not 32- or
    64-byte aligned for off = 16 or 48)."""

    def __init__(self, shape, dtype, off, init=None):
        t = torch()
        n = int(np.prod(shape)) * t.empty((), dtype=dtype).element_size()
        self.block = t.full((n + 512,), SENTINEL, dtype=t.uint8, device="cuda")
        base = self.block.data_ptr() % 256
        start = (256 - base) % 256 + off
        self.tensor = self.block[start:start + n].view(dtype).view(shape)
        assert self.tensor.data_ptr() % 256 == off
        if init is not None:
            src = t.from_numpy(np.ascontiguousarray(init).view(np.uint8).reshape(-1)).cuda()
            self.block[start:start + n].copy_(src)


@pytest.mark.parametrize("off", [16, 48])
@pytest.mark.parametrize("wbits", [4, 6, 8])
@pytest.mark.parametrize("paged", [False, True])
def test_sixteen_byte_aligned_buffers(kvq, off, wbits, paged):
    """Every buffer of a quantize + dequantize round trip 16 bytes past (or
    48 bytes past) a 256-byte boundary: the scalar whole-segment scale fetch
    of the Q4 / Q8 dequantize and every vector access must still read and
    write exactly the oracle's bytes.  Rows of 1024 elements (whole segments)
    and of 2048 in small launches, and rows of 1024 in launches of about
    9,000 units (two-unit quantize waves, runs of positions)."""
    t = torch()
    for head_dim, large in ((128, False), (256, False), (128, True)):
        rng = np.random.default_rng(off + wbits + head_dim + (7 if paged else 0) + (100 if large else 0))
        if paged:
            num_pages, ps, B, cols = (291, 16, 17, 17) if large else (9, 4, 3, 3)
            shape = (num_pages, ps, 8, head_dim)
            bt = rng.permutation(num_pages).astype(np.int32)[:B * cols].reshape(B, cols)
            sl = np.arange(B, dtype=np.int32) % 5 if large else np.array([0, 3, 5], np.int32)
            batch, offset, width = B, 0, (256 if large else 7)
            tabs = (ps, Offset(sl.shape, t.int32, off, sl).tensor, Offset(bt.shape, t.int32, off, bt).tensor)
            ref_tabs = (ps, sl, bt)
        else:
            shape = (3, 1500, 8, head_dim) if large else (3, 10, 8, head_dim)
            batch, offset, width = (3, 5, 1490) if large else (2, 3, 6)
            tabs = (0, None, None)
            ref_tabs = (0, None, None)
        k = (rng.standard_normal(shape) * 2).astype(np.float16)
        v = (rng.standard_normal(shape) * 0.5).astype(np.float16)
        gk, gv = Offset(shape, t.float16, off, k), Offset(shape, t.float16, off, v)
        gkq, gvq = Offset(_cs(shape, wbits), t.uint8, off), Offset(_cs(shape, wbits), t.uint8, off)
        gks, gvs = Offset(_ss(shape), t.float16, off), Offset(_ss(shape), t.float16, off)
        gko, gvo = Offset(shape, t.float16, off), Offset(shape, t.float16, off)
        kvq.kvq_fp16_to_q_kv(gk.tensor, gkq.tensor, gks.tensor, gv.tensor, gvq.tensor, gvs.tensor,
                             batch, offset, width, *tabs, wbits=wbits)
        kvq.kvq_q_to_fp16_kv(gkq.tensor, gko.tensor, gks.tensor, gvq.tensor, gvo.tensor, gvs.tensor,
                             batch, offset, width, *tabs, wbits=wbits)
        okq, ovq = sentinel_np(_cs(shape, wbits), np.uint8), sentinel_np(_cs(shape, wbits), np.uint8)
        oks, ovs = sentinel_np(_ss(shape), np.float16), sentinel_np(_ss(shape), np.float16)
        oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
        oracle.fp16_to_q_kv(k, okq, oks, v, ovq, ovs, batch, offset, width, *ref_tabs, wbits)
        oracle.q_to_fp16_kv(okq, oko, oks, ovq, ovo, ovs, batch, offset, width, *ref_tabs, wbits)
        what = "off %d Q%d %s head_dim %d%s" % (off, wbits, "paged" if paged else "contiguous", head_dim,
                                                 " large" if large else "")
        byte_diff(host(gkq.tensor), okq, what + " K codes")
        byte_diff(host(gvq.tensor), ovq, what + " V codes")
        byte_diff(host(gks.tensor), oks.view(np.uint16), what + " K scales")
        byte_diff(host(gvs.tensor), ovs.view(np.uint16), what + " V scales")
        byte_diff(host(gko.tensor), oko.view(np.uint16), what + " K out")
        byte_diff(host(gvo.tensor), ovo.view(np.uint16), what + " V out")


@pytest.mark.parametrize("off", [16, 48])
@pytest.mark.parametrize("fmts", [(4, 4), (4, 0), (8, 6), (8, 8)])
def test_sixteen_byte_aligned_per_tensor_and_prefix(kvq, off, fmts):
    """Per-tensor paged round trip and full-prefix widen (the uniform Q4 and
    Q8 pairs take the single-width kernels with the scalar scale fetch), and
    the contiguous 8-bit pair, with every buffer 16-byte aligned only."""
    t = torch()
    fk, fv = fmts
    rng = np.random.default_rng(off + 10 * fk + fv)
    num_pages, ps, B, cols = 9, 4, 3, 3
    shape = (num_pages, ps, 8, 128)
    bt = rng.permutation(num_pages).astype(np.int32)[:B * cols].reshape(B, cols)
    sl = np.array([1, 4, 2], np.int32)
    width, max_len = 6, cols * ps
    k = (rng.standard_normal(shape) * 2).astype(np.float16)
    v = (rng.standard_normal(shape) * 0.5).astype(np.float16)
    gsl, gbt = Offset(sl.shape, t.int32, off, sl).tensor, Offset(bt.shape, t.int32, off, bt).tensor
    gk, gv = Offset(shape, t.float16, off, k).tensor, Offset(shape, t.float16, off, v).tensor
    gkc, gvc = Offset(_cs(shape, fk), t.uint8, off).tensor, Offset(_cs(shape, fv), t.uint8, off).tensor
    gks = Offset(_ss(shape), t.float16, off).tensor if fk else None
    gvs = Offset(_ss(shape), t.float16, off).tensor if fv else None
    gko, gvo = Offset(shape, t.float16, off).tensor, Offset(shape, t.float16, off).tensor
    gpk, gpv = Offset(shape, t.float16, off).tensor, Offset(shape, t.float16, off).tensor
    a = (B, 0, width, ps, gsl, gbt)
    kvq.kvq_fp16_to_kv(gk, gkc, gks, fk, gv, gvc, gvs, fv, *a)
    kvq.kvq_kv_to_fp16(gkc, gko, gks, fk, gvc, gvo, gvs, fv, *a)
    kvq.kvq_kv_to_fp16_prefix(gkc, gpk, gks, fk, gvc, gpv, gvs, fv, B, width, max_len, gsl, gbt)
    okc, ovc = sentinel_np(_cs(shape, fk), np.uint8), sentinel_np(_cs(shape, fv), np.uint8)
    oks = sentinel_np(_ss(shape), np.float16) if fk else None
    ovs = sentinel_np(_ss(shape), np.float16) if fv else None
    oko, ovo = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    opk, opv = sentinel_np(shape, np.float16), sentinel_np(shape, np.float16)
    oracle.fp16_to_kv(k, okc, oks, fk, v, ovc, ovs, fv, B, 0, width, ps, sl, bt)
    oracle.kv_to_fp16(okc, oko, oks, fk, ovc, ovo, ovs, fv, B, 0, width, ps, sl, bt)
    oracle.kv_to_fp16_prefix(okc, opk, oks, fk, ovc, opv, ovs, fv, B, width, max_len, sl, bt)
    what = "off %d formats %s" % (off, fmts)
    byte_diff(host(gkc), okc, what + " K compact")
    byte_diff(host(gvc), ovc, what + " V compact")
    if fk:
        byte_diff(host(gks), oks.view(np.uint16), what + " K scales")
    if fv:
        byte_diff(host(gvs), ovs.view(np.uint16), what + " V scales")
    byte_diff(host(gko), oko.view(np.uint16), what + " K out")
    byte_diff(host(gvo), ovo.view(np.uint16), what + " V out")
    byte_diff(host(gpk), opk.view(np.uint16), what + " K prefix")
    byte_diff(host(gpv), opv.view(np.uint16), what + " V prefix")
    # contiguous 8-bit, window rows 1..5 of 2 sequences, on the same fp16 data
    cshape = (3, 12, 8, 128)
    x = (rng.standard_normal(cshape) * 3).astype(np.float16)
    gx = Offset(cshape, t.float16, off, x).tensor
    g8, gb = Offset(cshape, t.uint8, off).tensor, Offset(cshape, t.float16, off).tensor
    kvq.kvq_fp16_to_fp8(gx, g8, 2, 1, 5)
    kvq.kvq_fp8_to_fp16(g8, gb, 2, 1, 5)
    w8, wb = sentinel_np(cshape, np.uint8), sentinel_np(cshape, np.float16)
    oracle.fp16_to_fp8(x, w8, 2, 1, 5)
    oracle.fp8_to_fp16(w8, wb, 2, 1, 5)
    byte_diff(host(g8), w8, what + " 8-bit")
    byte_diff(host(gb), wb.view(np.uint16), what + " 8-bit back")
