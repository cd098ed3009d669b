"""Pins of the oracle's cache layouts, paged-row resolution and count_match.

The ExLlamaV2 cache page (Description, I/O Contract) fixes: contiguous
[batch, seq, heads, head_dim] caches converted over positions
[offset, offset + width) of each of batch_size sequences (a window of the
cache, outputs updated in place); paged mode when page_size > 0, with
block_table mapping logical to physical pages and cache_seqlens giving each
sequence's cache length; count_match counts how many leading elements two
1-D tensors share, up to max_a.

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import numpy as np
import pytest

import oracle

H, D = 2, 64                        # R = 128 elements per token row


def _sentinel_like(shape, dtype, byte=0xA5):
    a = np.empty(shape, dtype)
    a.view(np.uint8)[...] = byte
    return a


def _paged_positions(block_table_row, page_size, n_pos):
    """Expand one sequence's block table into (page, slot) for positions
    0..n_pos-1 by laying its pages end to end (enumeration, no division)."""
    out = []
    for page in block_table_row:
        for slot in range(page_size):
            out.append((int(page), slot))
            if len(out) == n_pos:
                return out
    return out + [None] * (n_pos - len(out))


@pytest.mark.parametrize("page_size", [1, 2, 3, 8])
def test_resolver_by_enumeration(page_size):
    rng = np.random.default_rng(page_size)
    dim0, cols, B = 40, 6, 3
    bt = rng.integers(-2, dim0 + 3, size=(B, cols)).astype(np.int32)   # some invalid pages
    sl = rng.integers(-3, cols * page_size, size=B).astype(np.int32)
    for offset in (0, 1, 2):
        width = cols * page_size + 2
        rows = oracle.call_rows(dim0, page_size, B, offset, width, page_size, sl, bt)
        for b in range(B):
            lay = _paged_positions(bt[b], page_size, cols * page_size)
            for t in range(width):
                p = int(sl[b]) + offset + t
                want = -1
                if 0 <= p < len(lay) and lay[p] is not None:
                    page, slot = lay[p]
                    if 0 <= page < dim0:
                        want = page * page_size + slot
                assert rows[b * width + t] == want, (b, t, p)


def test_contiguous_rows():
    rows = oracle.call_rows(5, 10, 3, 4, 5)
    want = [b * 10 + 4 + t for b in range(3) for t in range(5)]
    assert rows.tolist() == want


def _make_contig(rng, B, S):
    return (rng.standard_normal((B, S, H, D)) * 2).astype(np.float16)


@pytest.mark.parametrize("wbits", [4, 6])
def test_contiguous_window_and_untouched(wbits):
    rng = np.random.default_rng(21)
    B, S, offset, width, batch = 3, 20, 5, 7, 2
    k, v = _make_contig(rng, B, S), _make_contig(rng, B, S)
    cb = D * wbits // 8                 # code bytes per head
    kq, vq = _sentinel_like((B, S, H, cb), np.uint8), _sentinel_like((B, S, H, cb), np.uint8)
    ks, vs = _sentinel_like((B, S, H, D // 32), np.float16), _sentinel_like((B, S, H, D // 32), np.float16)
    oracle.fp16_to_q_kv(k, kq, ks, v, vq, vs, batch, offset, width, 0, None, None, wbits)
    inside = np.zeros((B, S), bool)
    inside[:batch, offset:offset + width] = True
    # rows outside the window keep their sentinel bytes
    assert (kq[~inside].view(np.uint8) == 0xA5).all() and (vs[~inside].view(np.uint8) == 0xA5).all()
    # rows inside equal the row-level quantization
    for x, q, s in ((k, kq, ks), (v, vq, vs)):
        c, sc = oracle.quant_rows(x[inside].reshape(-1, H * D), wbits)
        assert (q[inside].reshape(c.shape) == c).all()
        assert (s[inside].reshape(sc.shape).view(np.uint16) == sc).all()
    # dequantize back into a sentinel buffer: same window only
    ko = _sentinel_like((B, S, H, D), np.float16)
    oracle.q_to_fp16_kv(kq, ko, ks, None, None, None, batch, offset, width, 0, None, None, wbits)
    assert (ko[~inside].view(np.uint8) == 0xA5).all()
    want = oracle.dequant_rows(kq[inside].reshape(-1, H * cb), ks[inside].reshape(-1, H * D // 32), wbits)
    assert (ko[inside].reshape(-1, H * D).view(np.uint16) == want).all()
    # K and V in one call: each tensor is dequantized with its own scales
    # (the two tensors' scales differ: V is drawn independently of K)
    assert not np.array_equal(ks[inside].view(np.uint16), vs[inside].view(np.uint16))
    ko2, vo2 = _sentinel_like((B, S, H, D), np.float16), _sentinel_like((B, S, H, D), np.float16)
    oracle.q_to_fp16_kv(kq, ko2, ks, vq, vo2, vs, batch, offset, width, 0, None, None, wbits)
    for q, s, o in ((kq, ks, ko2), (vq, vs, vo2)):
        assert (o[~inside].view(np.uint8) == 0xA5).all()
        want = oracle.dequant_rows(q[inside].reshape(-1, H * cb), s[inside].reshape(-1, H * D // 32), wbits)
        assert (o[inside].reshape(-1, H * D).view(np.uint16) == want).all()


@pytest.mark.parametrize("wbits,page_size", [(4, 4), (6, 3), (4, 1)])
def test_paged_equals_contiguous(wbits, page_size):
    """Scatter a contiguous cache into pages through a permutation block
    table, quantize paged with cache_seqlens = start position, gather back:
    the bytes equal the contiguous run over the same window."""
    rng = np.random.default_rng(31 + page_size)
    B, S = 3, 24
    start, width = 5, 11
    cols = S // page_size
    num_pages = B * cols + 4
    k, v = _make_contig(rng, B, S), _make_contig(rng, B, S)
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = perm[:B * cols].reshape(B, cols)
    kp = np.zeros((num_pages, page_size, H, D), np.float16)
    vp = np.zeros_like(kp)
    for b in range(B):
        for p in range(S):
            kp[bt[b, p // page_size], p % page_size] = k[b, p]
            vp[bt[b, p // page_size], p % page_size] = v[b, p]
    cb = D * wbits // 8                 # code bytes per head
    # contiguous reference run
    kq = np.zeros((B, S, H, cb), np.uint8); vq = np.zeros_like(kq)
    ks = np.zeros((B, S, H, D // 32), np.float16); vs = np.zeros_like(ks)
    oracle.fp16_to_q_kv(k, kq, ks, v, vq, vs, B, start, width, 0, None, None, wbits)
    # paged run
    kqp = _sentinel_like((num_pages, page_size, H, cb), np.uint8); vqp = kqp.copy()
    ksp = _sentinel_like((num_pages, page_size, H, D // 32), np.float16); vsp = ksp.copy()
    sl = np.full(B, start, np.int32)
    oracle.fp16_to_q_kv(kp, kqp, ksp, vp, vqp, vsp, B, 0, width, page_size, sl, bt, wbits)
    touched = np.zeros((num_pages, page_size), bool)
    for b in range(B):
        for p in range(start, start + width):
            pg, sl_ = bt[b, p // page_size], p % page_size
            touched[pg, sl_] = True
            assert (kqp[pg, sl_] == kq[b, p]).all() and (vqp[pg, sl_] == vq[b, p]).all()
            assert (ksp[pg, sl_].view(np.uint16) == ks[b, p].view(np.uint16)).all()
            assert (vsp[pg, sl_].view(np.uint16) == vs[b, p].view(np.uint16)).all()
    assert (kqp[~touched] == 0xA5).all() and (vsp[~touched].view(np.uint8) == 0xA5).all()
    # K and V are independent: swapping the inputs swaps the outputs
    kq2 = np.zeros_like(kq); vq2 = np.zeros_like(vq); ks2 = np.zeros_like(ks); vs2 = np.zeros_like(vs)
    oracle.fp16_to_q_kv(v, kq2, ks2, k, vq2, vs2, B, start, width, 0, None, None, wbits)
    assert (kq2 == vq).all() and (vq2 == kq).all()
    assert (ks2.view(np.uint16) == vs.view(np.uint16)).all()


def test_paged_invalid_rows_skipped():
    wbits, page_size = 4, 2
    num_pages, cols, B = 6, 3, 2
    rng = np.random.default_rng(41)
    kp = (rng.standard_normal((num_pages, page_size, H, D))).astype(np.float16)
    bt = np.array([[1, -1, 7], [2, 3, 0]], np.int32)       # -1 and 7 are not pages
    sl = np.array([0, 5], np.int32)
    cb = D * wbits // 8                 # code bytes per head
    kq = _sentinel_like((num_pages, page_size, H, cb), np.uint8)
    ks = _sentinel_like((num_pages, page_size, H, D // 32), np.float16)
    oracle.fp16_to_q_kv(kp, kq, ks, None, None, None, B, 0, 4, page_size, sl, bt, wbits)
    # seq 0: p 0,1 -> page 1; p 2,3 -> page -1 (skipped)
    # seq 1: p 5 -> column 2 -> page 0 slot 1; p 6.. -> past the table (skipped)
    written = {(1, 0), (1, 1), (0, 1)}
    for pg in range(num_pages):
        for s in range(page_size):
            if (pg, s) in written:
                c, _ = oracle.quant_rows(kp[pg, s].reshape(1, -1), wbits)
                assert (kq[pg, s].reshape(-1) == c[0]).all()
            else:
                assert (kq[pg, s] == 0xA5).all()


def test_fp8_cache_window():
    rng = np.random.default_rng(51)
    B, S = 3, 9
    x = _make_contig(rng, B, S)
    out = _sentinel_like((B, S, H, D), np.uint8)
    oracle.fp16_to_fp8(x, out, 2, 3, 4)
    inside = np.zeros((B, S), bool)
    inside[:2, 3:7] = True
    assert (out[~inside] == 0xA5).all()
    assert (out[inside] == x[inside].view(np.uint8)[..., 1::2]).all()
    back = _sentinel_like((B, S, H, D), np.float16)
    oracle.fp8_to_fp16(out, back, 2, 3, 4)
    assert (back[~inside].view(np.uint8) == 0xA5).all()
    assert (back[inside].view(np.uint16) == (x[inside].view(np.uint16) & 0xFF00)).all()


# ---------------------------------------------------------------- count_match
@pytest.mark.parametrize("dtype", [np.int32, np.int64])
def test_count_match_planted(dtype):
    rng = np.random.default_rng(61)
    n = 1000
    a = rng.integers(0, 1 << 17, size=n).astype(dtype)
    for m in (0, 1, 7, 8, 9, 500, 999):
        b = a.copy()
        b[m] += 1
        for max_a in (0, 3, m, m + 1, n, n + 10):
            assert oracle.count_match(a, b, max_a) == min(m, max_a)
    assert oracle.count_match(a, a.copy(), n + 5) == n
    assert oracle.count_match(a, a[:10].copy(), n) == 10     # shorter b bounds it
    assert oracle.count_match(a, a.copy(), -3) == 0
    # elements are compared whole: a difference in any one byte is a mismatch
    for byte in range(np.dtype(dtype).itemsize):
        b = a.copy()
        b.view(np.uint8)[321 * b.itemsize + byte] ^= 0x40
        assert oracle.count_match(a, b, n) == 321


@pytest.mark.parametrize("dtype", [np.int32, np.int64])
def test_count_match_bruteforce_vs_numpy(dtype):
    rng = np.random.default_rng(62)
    for la in range(0, 18):
        for lb in range(0, 18, 3):
            a = rng.integers(0, 3, size=la).astype(dtype)
            b = rng.integers(0, 3, size=lb).astype(dtype)
            b[:min(la, lb) // 2] = a[:min(la, lb) // 2]
            for max_a in (la, 5, 100):
                n = max(0, min(max_a, la, lb))
                diff = np.nonzero(a[:n] != b[:n])[0]
                want = int(diff[0]) if diff.size else n
                assert oracle.count_match(a, b, max_a) == want


# ---------------------------------------------------------------- per-tensor formats, prefix, capacity
FMTS = (0, 4, 6, 8)


def _compact_np(shape, fmt):
    d0, d1, h, d = shape
    return _sentinel_like((d0, d1, h, d if fmt == 0 else d * fmt // 8), np.uint8)


def _scales_np(shape, fmt):
    if fmt == 0:
        return None
    d0, d1, h, d = shape
    return _sentinel_like((d0, d1, h, d // 32), np.float16)


def _paged_setup(rng, num_pages=20, page_size=4, B=3, cols=4):
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = perm[:B * cols].reshape(B, cols).copy()
    bt[1, 3] = -1                                    # an invalid entry
    sl = np.array([1, 6, 9], np.int32)[:B]
    return bt, sl


@pytest.mark.parametrize("fmt_k,fmt_v", [(0, 0), (0, 4), (4, 6), (6, 8), (8, 0)])
def test_per_tensor_formats_paged(fmt_k, fmt_v):
    """Each tensor in its own format equals the pinned single-format
    conversion of that tensor (block formats) or the fp16 memory image's high
    bytes (8-bit), on the rows the block-table expansion gives."""
    rng = np.random.default_rng(71 + fmt_k * 10 + fmt_v)
    page_size, num_pages, B, cols = 4, 20, 3, 4
    shape = (num_pages, page_size, H, D)
    k = (rng.standard_normal(shape) * 2).astype(np.float16)
    v = (rng.standard_normal(shape) * 0.3).astype(np.float16)
    bt, sl = _paged_setup(rng, num_pages, page_size, B, cols)
    width = 7
    kc, vc = _compact_np(shape, fmt_k), _compact_np(shape, fmt_v)
    ks, vs = _scales_np(shape, fmt_k), _scales_np(shape, fmt_v)
    oracle.fp16_to_kv(k, kc, ks, fmt_k, v, vc, vs, fmt_v, B, 0, width, page_size, sl, bt)
    touched = set()
    for b in range(B):
        lay = _paged_positions(bt[b], page_size, cols * page_size)
        for t in range(width):
            p = int(sl[b]) + t
            if p < len(lay) and lay[p] is not None and 0 <= lay[p][0] < num_pages:
                touched.add(lay[p])
    for x, c, sc, fmt in ((k, kc, ks, fmt_k), (v, vc, vs, fmt_v)):
        for pg in range(num_pages):
            for sl_ in range(page_size):
                if (pg, sl_) not in touched:
                    assert (c[pg, sl_] == 0xA5).all()
                    continue
                row = x[pg, sl_].reshape(1, -1)
                if fmt == 0:
                    assert (c[pg, sl_].reshape(-1) == row.view(np.uint8)[0, 1::2]).all()
                else:
                    codes, scales = oracle.quant_rows(row, fmt)
                    assert (c[pg, sl_].reshape(-1) == codes[0]).all()
                    assert (sc[pg, sl_].reshape(-1).view(np.uint16) == scales[0]).all()
    # and back
    ko, vo = _sentinel_like(shape, np.float16), _sentinel_like(shape, np.float16)
    oracle.kv_to_fp16(kc, ko, ks, fmt_k, vc, vo, vs, fmt_v, B, 0, width, page_size, sl, bt)
    for x, c, sc, o, fmt in ((k, kc, ks, ko, fmt_k), (v, vc, vs, vo, fmt_v)):
        for (pg, sl_) in touched:
            if fmt == 0:
                want = x[pg, sl_].reshape(-1).view(np.uint16) & 0xFF00
            else:
                want = oracle.dequant_rows(c[pg, sl_].reshape(1, -1), sc[pg, sl_].reshape(1, -1).view(np.uint16), fmt)[0]
            assert (o[pg, sl_].reshape(-1).view(np.uint16) == want).all()


def test_prefix_rows_by_enumeration():
    rng = np.random.default_rng(81)
    for page_size in (1, 3, 4):
        num_pages, B, cols = 30, 4, 5
        bt = rng.integers(-1, num_pages + 2, size=(B, cols)).astype(np.int32)
        sl = rng.integers(0, cols * page_size, size=B).astype(np.int32)
        for width, max_len in ((0, 100), (2, 100), (3, 7), (1, 0)):
            rows = oracle.prefix_rows(num_pages, page_size, B, width, max_len, sl, bt)
            want = []
            for b in range(B):
                lay = _paged_positions(bt[b], page_size, cols * page_size)
                for p in range(min(int(sl[b]) + width, max_len)):
                    ok = p < len(lay) and lay[p] is not None and 0 <= lay[p][0] < num_pages
                    want.append(lay[p][0] * page_size + lay[p][1] if ok else -1)
            assert rows.tolist() == want


@pytest.mark.parametrize("fmt", FMTS)
def test_prefix_widen_touches_exactly_the_prefix(fmt):
    rng = np.random.default_rng(91 + fmt)
    page_size, num_pages, B, cols = 4, 20, 3, 4
    shape = (num_pages, page_size, H, D)
    x = (rng.standard_normal(shape)).astype(np.float16)
    bt, sl = _paged_setup(rng, num_pages, page_size, B, cols)
    c, sc = _compact_np(shape, fmt), _scales_np(shape, fmt)
    # fill every row's compact form first (all rows valid input for widening)
    allrows = x.reshape(-1, H * D)
    if fmt == 0:
        c[...] = x.view(np.uint8)[..., 1::2]
    else:
        codes, scales = oracle.quant_rows(allrows, fmt)
        c.reshape(num_pages * page_size, -1)[...] = codes
        sc.reshape(num_pages * page_size, -1).view(np.uint16)[...] = scales
    out = _sentinel_like(shape, np.float16)
    width, max_len = 2, 14
    oracle.kv_to_fp16_prefix(c, out, sc, fmt, None, None, None, 0, B, width, max_len, sl, bt)
    rows = oracle.prefix_rows(num_pages, page_size, B, width, max_len, sl, bt)
    valid = set(int(r) for r in rows if r >= 0)
    flat_out = out.reshape(num_pages * page_size, -1).view(np.uint16)
    for r in range(num_pages * page_size):
        if r not in valid:
            assert (flat_out[r].view(np.uint8) == 0xA5).all()
        elif fmt == 0:
            assert (flat_out[r] == (allrows[r].view(np.uint16) & 0xFF00)).all()
        else:
            want = oracle.dequant_rows(c.reshape(num_pages * page_size, -1)[r:r + 1],
                                       sc.reshape(num_pages * page_size, -1)[r:r + 1].view(np.uint16), fmt)
            assert (flat_out[r] == want[0]).all()


@pytest.mark.parametrize("heads,head_dim", [(8, 128), (1, 32), (3, 96)])
def test_bytes_per_token_equals_output_sizes(heads, head_dim):
    R = heads * head_dim
    x = np.zeros((1, R), np.float16)
    assert oracle.bytes_per_token(16, heads, head_dim) == x.nbytes
    assert oracle.bytes_per_token(0, heads, head_dim) == x.view(np.uint8)[:, 1::2].nbytes
    for fmt in (4, 6, 8):
        codes, scales = oracle.quant_rows(x, fmt)
        assert oracle.bytes_per_token(fmt, heads, head_dim) == codes.nbytes + scales.nbytes
