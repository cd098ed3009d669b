"""CPU oracle for the KV-cache format conversions -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  It wraps ``kvq_oracle.c`` (plain scalar C, built with
gcc, IEEE arithmetic) through ctypes and operates on numpy arrays in host
memory.  It shares no code with the HIP library: the two sides only share the
seeded input generators, which hold none of the method's arithmetic.

The conventions each function follows are stated at the top of
``kvq_oracle.c``; the operations are the ones the page "Implementation:
Turboderp org Exllamav2 Ext Cache" lists (Description / Signature / I/O
Contract): fp16<->8-bit, fp16->Q4/Q6 with per-block fp16 scales for K and V,
the inverse, contiguous and paged layouts, and the host prefix compare.  It
also covers the extensions built on them: block Q8 (the page's Usage section
lists a Q8 cache class), a format per tensor (8-bit on paged caches, K and V
at different widths), the full-prefix widen before attention, and the bytes
per token of each format.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def lib():
    """Load (building once if absent) the oracle shared library.  The
    environment variable KVQ_ORACLE_LIB names another build of kvq_oracle.c
    to load instead; the mutation test uses it to run the pins against
    builds with planted mistakes."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("KVQ_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        sig = {
            "orc_f16_decode": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_f16_encode_rne": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_fp8_from_f16": (ctypes.c_uint8, [ctypes.c_uint16]),
            "orc_f16_from_fp8": (ctypes.c_uint16, [ctypes.c_uint8]),
            "orc_scale_from_absmax": (ctypes.c_uint16, [ctypes.c_uint16, _int]),
            "orc_quant_elems": (None, [_u16p, _i64, ctypes.c_uint16, _int, _u8p]),
            "orc_quant_block": (None, [_u16p, _int, _int, _u16p, _u8p]),
            "orc_dequant_elems": (None, [_u8p, _i64, ctypes.c_uint16, _int, _u16p]),
            "orc_pack_bits": (None, [_u8p, _i64, _int, _u8p]),
            "orc_unpack_bits": (None, [_u8p, _i64, _int, _u8p]),
            "orc_quant_rows": (None, [_u16p, _i64, _int, _int, _u8p, _u16p]),
            "orc_dequant_rows": (None, [_u8p, _u16p, _i64, _int, _int, _u16p]),
            "orc_resolve_row": (_i64, [_int, _int, _int, _int, _int, _int, _i32p, _i32p, _int]),
            "orc_call_rows": (_i64, [_int, _int, _int, _int, _int, _int, _i32p, _i32p, _int, _i64p]),
            "orc_fp16_to_q_kv": (None, [_u16p, _u8p, _u16p, _u16p, _u8p, _u16p,
                                        _int, _int, _int, _int, _int, _int, _int, _int,
                                        _i32p, _i32p, _int, _int]),
            "orc_q_to_fp16_kv": (None, [_u8p, _u16p, _u16p, _u8p, _u16p, _u16p,
                                        _int, _int, _int, _int, _int, _int, _int, _int,
                                        _i32p, _i32p, _int, _int]),
            "orc_fp16_to_fp8_cache": (None, [_u16p, _u8p, _int, _int, _int, _int, _int, _int, _int]),
            "orc_fp8_to_fp16_cache": (None, [_u8p, _u16p, _int, _int, _int, _int, _int, _int, _int]),
            "orc_count_match": (_i64, [ctypes.c_void_p, _i64, ctypes.c_void_p, _i64, _i64, _int]),
            "orc_fp16_to_kv": (None, [_u16p, _u8p, _u16p, _int, _u16p, _u8p, _u16p, _int,
                                      _int, _int, _int, _int, _int, _int, _int, _int,
                                      _i32p, _i32p, _int]),
            "orc_kv_to_fp16": (None, [_u8p, _u16p, _u16p, _int, _u8p, _u16p, _u16p, _int,
                                      _int, _int, _int, _int, _int, _int, _int, _int,
                                      _i32p, _i32p, _int]),
            "orc_prefix_rows": (_i64, [_int, _int, _int, _int, _int, _i32p, _i32p, _int, _i64p]),
            "orc_kv_to_fp16_prefix": (None, [_u8p, _u16p, _u16p, _int, _u8p, _u16p, _u16p, _int,
                                             _int, _int, _int, _int, _int, _int, _int,
                                             _i32p, _i32p, _int]),
            "orc_bytes_per_token": (_i64, [_int, _int, _int]),
            "orc_f16_decode_array": (None, [_u16p, _i64, _f64p]),
            "orc_f16_encode_array": (None, [_f64p, _i64, _u16p]),
            "orc_scale_array": (None, [_u16p, _i64, _int, _u16p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _p(arr, ptype):
    """ctypes pointer to a C-contiguous numpy array (or NULL for None)."""
    if arr is None:
        return ctypes.cast(None, ptype)
    assert arr.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return arr.ctypes.data_as(ptype)


def _as_u16(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a.astype(np.uint16, copy=False)


# ---------------------------------------------------------------- fp16 codec
def f16_decode(bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().orc_f16_decode_array(_p(bits.ravel(), _u16p), bits.size, _p(out.reshape(-1), _f64p))
    return out


def f16_encode_rne(values):
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_f16_encode_array(_p(v.ravel(), _f64p), v.size, _p(out.reshape(-1), _u16p))
    return out


# ---------------------------------------------------------------- 8-bit
def fp8_from_f16(bits):
    L = lib()
    return np.array([L.orc_fp8_from_f16(int(h)) for h in np.asarray(bits, np.uint16).ravel()],
                    np.uint8).reshape(np.shape(bits))


def f16_from_fp8(b):
    L = lib()
    return np.array([L.orc_f16_from_fp8(int(x)) for x in np.asarray(b, np.uint8).ravel()],
                    np.uint16).reshape(np.shape(b))


# ---------------------------------------------------------------- block quantization
def scale_from_absmax(a_bits, wbits):
    a = np.ascontiguousarray(a_bits, dtype=np.uint16)
    out = np.empty(a.shape, np.uint16)
    lib().orc_scale_array(_p(a.ravel(), _u16p), a.size, wbits, _p(out.reshape(-1), _u16p))
    return out


def quant_elems(x_bits, s16, wbits):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    u = np.empty(x.shape, np.uint8)
    lib().orc_quant_elems(_p(x.ravel(), _u16p), x.size, int(s16), wbits, _p(u.reshape(-1), _u8p))
    return u


def quant_block(x_bits, wbits):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    u = np.empty(x.shape, np.uint8)
    s = np.zeros(1, np.uint16)
    lib().orc_quant_block(_p(x, _u16p), x.size, wbits, _p(s, _u16p), _p(u, _u8p))
    return int(s[0]), u


def dequant_elems(u, s16, wbits):
    u = np.ascontiguousarray(u, dtype=np.uint8)
    out = np.empty(u.shape, np.uint16)
    lib().orc_dequant_elems(_p(u.ravel(), _u8p), u.size, int(s16), wbits, _p(out.reshape(-1), _u16p))
    return out


def pack_bits(u, wbits):
    u = np.ascontiguousarray(u, dtype=np.uint8)
    out = np.empty((u.size * wbits + 7) // 8, np.uint8)
    lib().orc_pack_bits(_p(u, _u8p), u.size, wbits, _p(out, _u8p))
    return out


def unpack_bits(packed, n, wbits):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    u = np.empty(n, np.uint8)
    lib().orc_unpack_bits(_p(packed, _u8p), n, wbits, _p(u, _u8p))
    return u


# ---------------------------------------------------------------- token rows
def quant_rows(rows_f16, wbits):
    """rows: [n, R] fp16 (or uint16 bits) -> (codes [n, R*wbits/8] u8, scales [n, R/32] u16)."""
    x = _as_u16(rows_f16)
    n, R = x.shape
    codes = np.empty((n, R * wbits // 8), np.uint8)
    scales = np.empty((n, R // 32), np.uint16)
    lib().orc_quant_rows(_p(x, _u16p), n, R, wbits, _p(codes, _u8p), _p(scales, _u16p))
    return codes, scales


def dequant_rows(codes, scales, wbits):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = _as_u16(scales)
    n = codes.shape[0]
    R = scales.shape[1] * 32
    out = np.empty((n, R), np.uint16)
    lib().orc_dequant_rows(_p(codes, _u8p), _p(scales, _u16p), n, R, wbits, _p(out, _u16p))
    return out


# ---------------------------------------------------------------- cache level
def _meta(cache_seqlens, block_table):
    sl = None if cache_seqlens is None else np.ascontiguousarray(cache_seqlens, np.int32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, np.int32)
    cols = 0 if bt is None else (bt.shape[1] if bt.ndim == 2 else bt.size)
    return sl, bt, cols


def call_rows(dim0, dim1, batch_size, offset, width, page_size=0,
              cache_seqlens=None, block_table=None):
    """Flat physical row index of every (b, t) of a call, -1 where skipped."""
    sl, bt, cols = _meta(cache_seqlens, block_table)
    rows = np.empty(max(batch_size * width, 1), np.int64)
    n = lib().orc_call_rows(dim0, dim1, batch_size, offset, width, page_size,
                            _p(sl, _i32p), _p(bt, _i32p), cols, _p(rows, _i64p))
    return rows[:n]


def fp16_to_q_kv(k_in, k_out, k_scales, v_in, v_out, v_scales, batch_size, offset, width,
                 page_size, cache_seqlens, block_table, wbits):
    """In place on host arrays shaped like the library's (see kvq.h)."""
    ref = k_in if k_in is not None else v_in
    dim0, dim1, heads, head_dim = ref.shape
    sl, bt, cols = _meta(cache_seqlens, block_table)
    lib().orc_fp16_to_q_kv(
        _p(None if k_in is None else _as_u16(k_in), _u16p), _p(k_out, _u8p),
        _p(None if k_scales is None else k_scales.view(np.uint16), _u16p),
        _p(None if v_in is None else _as_u16(v_in), _u16p), _p(v_out, _u8p),
        _p(None if v_scales is None else v_scales.view(np.uint16), _u16p),
        dim0, dim1, heads, head_dim, batch_size, offset, width, page_size,
        _p(sl, _i32p), _p(bt, _i32p), cols, wbits)


def q_to_fp16_kv(k_in, k_out, k_scales, v_in, v_out, v_scales, batch_size, offset, width,
                 page_size, cache_seqlens, block_table, wbits):
    ref = k_out if k_out is not None else v_out
    dim0, dim1, heads, head_dim = ref.shape
    sl, bt, cols = _meta(cache_seqlens, block_table)
    lib().orc_q_to_fp16_kv(
        _p(k_in, _u8p), _p(None if k_out is None else k_out.view(np.uint16), _u16p),
        _p(None if k_scales is None else _as_u16(k_scales), _u16p),
        _p(v_in, _u8p), _p(None if v_out is None else v_out.view(np.uint16), _u16p),
        _p(None if v_scales is None else _as_u16(v_scales), _u16p),
        dim0, dim1, heads, head_dim, batch_size, offset, width, page_size,
        _p(sl, _i32p), _p(bt, _i32p), cols, wbits)


def fp16_to_fp8(x, out, batch_size, offset, width):
    dim0, dim1, heads, head_dim = x.shape
    lib().orc_fp16_to_fp8_cache(_p(_as_u16(x), _u16p), _p(out, _u8p), dim0, dim1, heads, head_dim,
                                batch_size, offset, width)


def fp8_to_fp16(x, out, batch_size, offset, width):
    dim0, dim1, heads, head_dim = x.shape
    lib().orc_fp8_to_fp16_cache(_p(x, _u8p), _p(out.view(np.uint16), _u16p), dim0, dim1, heads,
                                head_dim, batch_size, offset, width)


def count_match(a, b, max_a):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.dtype == b.dtype and a.itemsize in (4, 8)
    return int(lib().orc_count_match(a.ctypes.data, a.size, b.ctypes.data, b.size, int(max_a),
                                     a.itemsize))


# ---------------------------------------------------------------- per-tensor formats
# fmt 0 = 8-bit high byte (no scales); 4, 6, 8 = block codes + fp16 scales.
def _u16(a):
    return None if a is None else (a.view(np.uint16) if a.dtype == np.float16 else a)


def fp16_to_kv(k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, batch_size, offset,
               width, page_size=0, cache_seqlens=None, block_table=None):
    ref = k_in if k_in is not None else v_in
    dim0, dim1, heads, head_dim = ref.shape
    sl, bt, cols = _meta(cache_seqlens, block_table)
    lib().orc_fp16_to_kv(
        _p(None if k_in is None else _as_u16(k_in), _u16p), _p(k_out, _u8p), _p(_u16(k_scales), _u16p), fmt_k,
        _p(None if v_in is None else _as_u16(v_in), _u16p), _p(v_out, _u8p), _p(_u16(v_scales), _u16p), fmt_v,
        dim0, dim1, heads, head_dim, batch_size, offset, width, page_size, _p(sl, _i32p), _p(bt, _i32p), cols)


def kv_to_fp16(k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, batch_size, offset,
               width, page_size=0, cache_seqlens=None, block_table=None):
    ref = k_out if k_out is not None else v_out
    dim0, dim1, heads, head_dim = ref.shape
    sl, bt, cols = _meta(cache_seqlens, block_table)
    lib().orc_kv_to_fp16(
        _p(k_in, _u8p), _p(_u16(k_out), _u16p), _p(_u16(k_scales), _u16p), fmt_k,
        _p(v_in, _u8p), _p(_u16(v_out), _u16p), _p(_u16(v_scales), _u16p), fmt_v,
        dim0, dim1, heads, head_dim, batch_size, offset, width, page_size, _p(sl, _i32p), _p(bt, _i32p), cols)


def prefix_rows(dim0, page_size, batch_size, width, max_len, cache_seqlens, block_table):
    """Physical rows of positions [0, min(cache_seqlens[b] + width, max_len))
    of every sequence, in (b, p) order, -1 where skipped."""
    sl, bt, cols = _meta(cache_seqlens, block_table)
    total = int(sum(max(0, min(int(x) + width, max_len)) for x in sl))
    rows = np.empty(max(total, 1), np.int64)
    n = lib().orc_prefix_rows(dim0, page_size, batch_size, width, max_len, _p(sl, _i32p), _p(bt, _i32p),
                              cols, _p(rows, _i64p))
    return rows[:n]


def kv_to_fp16_prefix(k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, batch_size, width,
                      max_len, cache_seqlens, block_table):
    ref = k_out if k_out is not None else v_out
    dim0, dim1, heads, head_dim = ref.shape
    sl, bt, cols = _meta(cache_seqlens, block_table)
    lib().orc_kv_to_fp16_prefix(
        _p(k_in, _u8p), _p(_u16(k_out), _u16p), _p(_u16(k_scales), _u16p), fmt_k,
        _p(v_in, _u8p), _p(_u16(v_out), _u16p), _p(_u16(v_scales), _u16p), fmt_v,
        dim0, dim1, heads, head_dim, batch_size, width, max_len, _p(sl, _i32p), _p(bt, _i32p), cols)


def bytes_per_token(fmt, heads, head_dim):
    return int(lib().orc_bytes_per_token(fmt, heads, head_dim))
