"""Pins of the oracle's cache layouts, paged-row resolution and count_match.

The ExLlamaV2 cache page (Description, I/O Contract) fixes: contiguous
[batch, seq, heads, head_dim] caches converted over positions
[offset, offset + width) of each of batch_size sequences ("partial cache
updates", results written in place); paged mode when page_size > 0, with
block_table mapping logical to physical pages and cache_seqlens giving each
sequence's cache length; count_match returns the length of the matching
prefix of two 1-D tensors, at most max_a.
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
