"""kvq -- KV-cache format conversion on MI355X (gfx950).

Thin ctypes binding over the C ABI in include/kvq.h (libkvq.so, built in-tree
by ``_build.build()``).  Each function has the name of its C entry point and
only marshals arguments: dtype / shape / device checks on torch tensors,
pointers, the current HIP stream.  Every step of the conversion runs in the
HIP kernels; there is no fallback.  If the library has not been built, the
first call raises.

Operations (ExLlamaV2 cache page, Description / Signature / I/O Contract):
  kvq_fp16_to_fp8 / kvq_fp8_to_fp16    fp16 <-> 8-bit (fp16 high byte)
  kvq_fp16_to_q_kv / kvq_q_to_fp16_kv  fp16 <-> 4/6-bit block codes + fp16
                                       scales, K and V in one launch,
                                       contiguous or paged
  kvq_count_match                      host matching-prefix length

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import ctypes
import os

from . import _build

__all__ = ["KvqError", "kvq_fp16_to_fp8", "kvq_fp8_to_fp16", "kvq_fp16_to_q_kv",
           "kvq_q_to_fp16_kv", "kvq_count_match", "kvq_strerror", "kvq_version",
           "kvq_selftest_codes", "kvq_selftest_scales", "kvq_selftest_fastdiv", "kvq_selftest_copy", "kvq_selftest_stream", "library_path", "load_library",
           "code_shape", "scale_shape", "kvq_fp16_to_kv", "kvq_kv_to_fp16", "kvq_kv_to_fp16_prefix",
           "kvq_bytes_per_token", "compact_shape", "KVQ_FMT_FP8", "KVQ_FMT_Q4", "KVQ_FMT_Q6",
           "KVQ_FMT_Q8", "KVQ_FMT_FP16"]

# per-tensor formats (include/kvq.h)
KVQ_FMT_FP8, KVQ_FMT_Q4, KVQ_FMT_Q6, KVQ_FMT_Q8, KVQ_FMT_FP16 = 0, 4, 6, 8, 16

KVQ_OK = 0
ERRORS = {-1: "KVQ_ERR_NULL", -2: "KVQ_ERR_WBITS", -3: "KVQ_ERR_SHAPE", -4: "KVQ_ERR_RANGE",
          -5: "KVQ_ERR_ALIGN", -6: "KVQ_ERR_OVERLAP", -7: "KVQ_ERR_HIP"}


class KvqError(RuntimeError):
    def __init__(self, code, fn):
        self.code = code
        super().__init__("%s failed: %s (%s)" % (fn, ERRORS.get(code, code), kvq_strerror(code)))


class Shape(ctypes.Structure):
    _fields_ = [("dim0", ctypes.c_int32), ("dim1", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


_LIB = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64


def library_path():
    return _build.LIB


def load_library():
    """Load libkvq.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(
                "libkvq.so is not built (%s); run kv_cache_quantization_kvq_amd._build.build()"
                % _build.LIB)
        # torch ships its own HIP runtime (libamdhip64, same soname as the
        # system one libkvq.so is linked against).  Loading torch first makes
        # the library bind to that runtime; loaded the other way round, the
        # process would hold two HIP runtimes, and the tensors and streams the
        # binding passes would belong to the one the kernels are not launched on.
        _torch()
        L = ctypes.CDLL(_build.LIB)
        q_args = [_vp, _vp, _vp, _vp, _vp, _vp, Shape, _i, _i, _i, _i, _vp, _vp, _i, _i, _vp]
        sig = {
            "kvq_fp16_to_fp8": (_i, [_vp, _vp, Shape, _i, _i, _i, _vp]),
            "kvq_fp8_to_fp16": (_i, [_vp, _vp, Shape, _i, _i, _i, _vp]),
            "kvq_fp16_to_q_kv": (_i, q_args),
            "kvq_q_to_fp16_kv": (_i, q_args),
            "kvq_count_match": (_i64, [_vp, _i64, _vp, _i64, _i64, _i]),
            "kvq_strerror": (ctypes.c_char_p, [_i]),
            "kvq_version": (_i, []),
            "kvq_selftest_codes": (_i, [_vp, _i64, _vp, _i64, _i, _i, _vp, _vp]),
            "kvq_selftest_scales": (_i, [_vp, _i64, _i, _vp, _vp]),
            "kvq_selftest_fastdiv": (_i, [_vp, _i64, ctypes.c_uint32, _vp, _vp]),
            "kvq_selftest_copy": (_i, [_vp, _vp, _i64, _i, _i, _i64, _vp]),
            "kvq_selftest_stream": (_i, [_vp, _i64, _vp, _i64, _i, _i, _vp]),
            "kvq_fp16_to_kv": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, Shape, _i, _i, _i, _i,
                                    _vp, _vp, _i, _vp]),
            "kvq_kv_to_fp16": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, Shape, _i, _i, _i, _i,
                                    _vp, _vp, _i, _vp]),
            "kvq_kv_to_fp16_prefix": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, Shape, _i, _i, _i,
                                           _vp, _vp, _i, _vp]),
            "kvq_bytes_per_token": (_i64, [_i, _i, _i]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def kvq_strerror(code):
    return load_library().kvq_strerror(int(code)).decode()


def kvq_version():
    return load_library().kvq_version()


# ---------------------------------------------------------------- marshalling helpers
#
# These run on every call, so they keep the per-call Python work small: the
# torch module and the current-stream query are looked up once, devices are
# compared by index, and the full diagnosis (which check failed) is only
# made once a check has failed.

_TORCH = None
_RAW_STREAM = None
_SHAPES = {}


def _torch():
    global _TORCH, _RAW_STREAM
    if _TORCH is None:
        import torch
        # the current stream's raw handle of a device index, without building
        # a Stream object (the public query is the fallback)
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _TORCH = torch
    return _TORCH


def _check(rc, fn):
    if rc != KVQ_OK:
        raise KvqError(rc, fn)


def _shape_struct(shp):
    st = _SHAPES.get(shp)
    if st is None:
        if len(_SHAPES) >= 256:
            _SHAPES.clear()
        st = _SHAPES[shp] = Shape(*shp)
    return st


def _dev_ptr(t, name, dtype, device=None):
    """Device address of a contiguous tensor of `dtype` (None passes through);
    `device` is a device index the tensor must be on, or None."""
    if t is None:
        return None
    torch = _TORCH or _torch()
    if (isinstance(t, torch.Tensor) and t.dtype is dtype and t.is_cuda and t.is_contiguous()
            and (device is None or t.get_device() == device)):
        return t.data_ptr()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if device is not None and t.get_device() != device:
        raise ValueError("%s is on %s, expected cuda:%d" % (name, t.device, device))
    raise ValueError("%s must be contiguous" % name)


def _table_ptr(t, name, device):
    if t is None:
        return None
    return _dev_ptr(t, name, _torch().int32, device)


def _stream_handle(stream, device):
    """Raw HIP stream handle: `stream` (a torch stream or a handle), or the
    current stream of device index `device`."""
    if stream is None:
        torch = _TORCH or _torch()
        if _RAW_STREAM is not None:
            return _RAW_STREAM(device)
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _expect_shape(t, shape, name):
    if t is not None and t.shape != shape:
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def code_shape(cache_shape, wbits):
    d0, d1, h, d = cache_shape
    return (d0, d1, h, d * wbits // 8)


def scale_shape(cache_shape):
    d0, d1, h, d = cache_shape
    return (d0, d1, h, d // 32)


def _shape4(t, name):
    if t.dim() != 4:
        raise ValueError("%s must be 4-D [dim0, dim1, heads, head_dim]" % name)
    return tuple(t.shape)


def _device_of(t):
    """Device index of a device tensor (-1 for host tensors, which the
    pointer checks then reject)."""
    return t.get_device()


# ---------------------------------------------------------------- 8-bit
def kvq_fp16_to_fp8(in_tensor, out_tensor, batch_size, offset, width, stream=None):
    """fp16 cache -> uint8 cache (high byte), rows (b, offset + t) of the
    window, b < batch_size, t < width.  Asynchronous on `stream`."""
    torch = _torch()
    shp = _shape4(in_tensor, "in_tensor")
    pi = _dev_ptr(in_tensor, "in_tensor", torch.float16)
    dev = _device_of(in_tensor)
    po = _dev_ptr(out_tensor, "out_tensor", torch.uint8, dev)
    _expect_shape(out_tensor, shp, "out_tensor")
    rc = load_library().kvq_fp16_to_fp8(pi, po, _shape_struct(shp), int(batch_size), int(offset),
                                        int(width), _stream_handle(stream, dev))
    _check(rc, "kvq_fp16_to_fp8")


def kvq_fp8_to_fp16(in_tensor, out_tensor, batch_size, offset, width, stream=None):
    """uint8 cache -> fp16 cache (byte << 8) over the same window."""
    torch = _torch()
    shp = _shape4(in_tensor, "in_tensor")
    pi = _dev_ptr(in_tensor, "in_tensor", torch.uint8)
    dev = _device_of(in_tensor)
    po = _dev_ptr(out_tensor, "out_tensor", torch.float16, dev)
    _expect_shape(out_tensor, shp, "out_tensor")
    rc = load_library().kvq_fp8_to_fp16(pi, po, _shape_struct(shp), int(batch_size), int(offset),
                                        int(width), _stream_handle(stream, dev))
    _check(rc, "kvq_fp8_to_fp16")


# ---------------------------------------------------------------- 4/6-bit K/V
def _q_common(quant, k_in, k_out, k_scales, v_in, v_out, v_scales, batch_size, offset, width,
              page_size, cache_seqlens, block_table, wbits, stream):
    torch = _torch()
    fname = "kvq_fp16_to_q_kv" if quant else "kvq_q_to_fp16_kv"
    f16 = k_in if quant else k_out
    f16v = v_in if quant else v_out
    ref = f16 if f16 is not None else f16v
    if ref is None:
        raise ValueError("%s: at least one of the K and V triples is required" % fname)
    shp = _shape4(ref, "cache")
    dev = _device_of(ref)
    if wbits not in (4, 6, 8):
        raise ValueError("wbits must be 4, 6 or 8")
    cshape, sshape = code_shape(shp, wbits), scale_shape(shp)
    src_t, dst_t = (torch.float16, torch.uint8) if quant else (torch.uint8, torch.float16)
    src_s, dst_s = (shp, cshape) if quant else (cshape, shp)
    ptrs = []
    for nm, t, dt, sh in (("k_in", k_in, src_t, src_s), ("k_out", k_out, dst_t, dst_s),
                          ("k_scales", k_scales, torch.float16, sshape),
                          ("v_in", v_in, src_t, src_s), ("v_out", v_out, dst_t, dst_s),
                          ("v_scales", v_scales, torch.float16, sshape)):
        ptrs.append(_dev_ptr(t, nm, dt, dev))
        _expect_shape(t, sh, nm)
    cols = 0
    psl = pbt = None
    if page_size:
        if cache_seqlens is None or block_table is None:
            raise ValueError("paged mode needs cache_seqlens and block_table")
        if block_table.dim() != 2 or block_table.shape[0] < batch_size:
            raise ValueError("block_table must be [>= batch_size, cols]")
        if cache_seqlens.dim() != 1 or cache_seqlens.shape[0] < batch_size:
            raise ValueError("cache_seqlens must be [>= batch_size]")
        cols = int(block_table.shape[1])
        psl = _table_ptr(cache_seqlens, "cache_seqlens", dev)
        pbt = _table_ptr(block_table, "block_table", dev)
    fn = getattr(load_library(), fname)
    rc = fn(*ptrs, _shape_struct(shp), int(batch_size), int(offset), int(width), int(page_size),
            psl, pbt, cols, int(wbits), _stream_handle(stream, dev))
    _check(rc, fname)


def kvq_fp16_to_q_kv(k_in, k_out, k_scales, v_in, v_out, v_scales, batch_size, offset, width,
                     page_size=0, cache_seqlens=None, block_table=None, wbits=4, stream=None):
    """fp16 K/V caches -> codes [dim0, dim1, heads, head_dim*wbits/8] (uint8)
    and scales [dim0, dim1, heads, head_dim/32] (fp16).  Pass None for a
    whole triple to skip that half.  page_size > 0 selects the paged layout
    (then cache_seqlens: int32[batch], block_table: int32[batch, cols])."""
    _q_common(True, k_in, k_out, k_scales, v_in, v_out, v_scales, batch_size, offset, width,
              page_size, cache_seqlens, block_table, wbits, stream)


def kvq_q_to_fp16_kv(k_in, k_out, k_scales, v_in, v_out, v_scales, batch_size, offset, width,
                     page_size=0, cache_seqlens=None, block_table=None, wbits=4, stream=None):
    """codes + scales -> fp16 K/V caches over the same rows (k_in/v_in are the
    codes, k_out/v_out the fp16 caches)."""
    _q_common(False, k_in, k_out, k_scales, v_in, v_out, v_scales, batch_size, offset, width,
              page_size, cache_seqlens, block_table, wbits, stream)


# ---------------------------------------------------------------- per-tensor formats
def compact_shape(cache_shape, fmt):
    """Shape of a tensor's compact form: uint8 of the cache shape for the
    8-bit format, the code shape for the block formats."""
    return tuple(cache_shape) if fmt == KVQ_FMT_FP8 else code_shape(cache_shape, fmt)


def _kv_ptrs(to_compact, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v):
    torch = _torch()
    ref = None
    for t in ((k_in, v_in) if to_compact else (k_out, v_out)):
        if t is not None:
            ref = t
            break
    if ref is None:
        raise ValueError("at least one of K and V is required")
    shp = _shape4(ref, "cache")
    dev = _device_of(ref)
    ptrs = []
    for name, (src, dst, sc, fmt) in (("k", (k_in, k_out, k_scales, fmt_k)), ("v", (v_in, v_out, v_scales, fmt_v))):
        if src is None and dst is None:
            ptrs += [None, None, _dev_ptr(sc, name + "_scales", torch.float16, dev) if sc is not None else None]
            continue
        if fmt not in (0, 4, 6, 8):
            raise ValueError("%s format must be KVQ_FMT_FP8, Q4, Q6 or Q8" % name)
        cshape = compact_shape(shp, fmt)
        f16, comp = (src, dst) if to_compact else (dst, src)
        pf16 = _dev_ptr(f16, name + " fp16 cache", torch.float16, dev)
        pcomp = _dev_ptr(comp, name + " compact cache", torch.uint8, dev)
        _expect_shape(f16, shp, name + " fp16 cache")
        _expect_shape(comp, cshape, name + " compact cache")
        psc = None
        if sc is not None:
            psc = _dev_ptr(sc, name + "_scales", torch.float16, dev)
            _expect_shape(sc, scale_shape(shp), name + "_scales")
        ptrs += ([pf16, pcomp, psc] if to_compact else [pcomp, pf16, psc])
    return ptrs, shp, dev


def _tables(batch_size, cache_seqlens, block_table, dev):
    if block_table.dim() != 2 or block_table.shape[0] < batch_size:
        raise ValueError("block_table must be [>= batch_size, cols]")
    if cache_seqlens.dim() != 1 or cache_seqlens.shape[0] < batch_size:
        raise ValueError("cache_seqlens must be [>= batch_size]")
    return (_table_ptr(cache_seqlens, "cache_seqlens", dev), _table_ptr(block_table, "block_table", dev),
            int(block_table.shape[1]))


def _per_tensor(fname, to_compact, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v,
                batch_size, offset, width, page_size, cache_seqlens, block_table, stream):
    ptrs, shp, dev = _kv_ptrs(to_compact, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v)
    psl = pbt = None
    cols = 0
    if page_size:
        if cache_seqlens is None or block_table is None:
            raise ValueError("paged mode needs cache_seqlens and block_table")
        psl, pbt, cols = _tables(batch_size, cache_seqlens, block_table, dev)
    rc = getattr(load_library(), fname)(ptrs[0], ptrs[1], ptrs[2], int(fmt_k), ptrs[3], ptrs[4], ptrs[5],
                                        int(fmt_v), _shape_struct(shp), int(batch_size), int(offset), int(width),
                                        int(page_size), psl, pbt, cols, _stream_handle(stream, dev))
    _check(rc, fname)


def kvq_fp16_to_kv(k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, batch_size, offset,
                   width, page_size=0, cache_seqlens=None, block_table=None, stream=None):
    """fp16 K/V -> per-tensor formats in one launch (KVQ_FMT_FP8: uint8 cache,
    no scales; KVQ_FMT_Q4/Q6/Q8: codes + fp16 scales).  Pass None for the
    three tensors of an absent half."""
    _per_tensor("kvq_fp16_to_kv", True, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v,
                batch_size, offset, width, page_size, cache_seqlens, block_table, stream)


def kvq_kv_to_fp16(k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, batch_size, offset,
                   width, page_size=0, cache_seqlens=None, block_table=None, stream=None):
    """Per-tensor formats -> fp16 K/V in one launch over the same rows."""
    _per_tensor("kvq_kv_to_fp16", False, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v,
                batch_size, offset, width, page_size, cache_seqlens, block_table, stream)


def kvq_kv_to_fp16_prefix(k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, batch_size,
                          width, max_len, cache_seqlens, block_table, stream=None):
    """Widen positions [0, min(cache_seqlens[b] + width, max_len)) of every
    sequence of a paged cache (page_size = the caches' dim 1)."""
    ptrs, shp, dev = _kv_ptrs(False, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v)
    psl, pbt, cols = _tables(batch_size, cache_seqlens, block_table, dev)
    rc = load_library().kvq_kv_to_fp16_prefix(ptrs[0], ptrs[1], ptrs[2], int(fmt_k), ptrs[3], ptrs[4],
                                              ptrs[5], int(fmt_v), _shape_struct(shp), int(batch_size),
                                              int(width), int(max_len), psl, pbt, cols,
                                              _stream_handle(stream, dev))
    _check(rc, "kvq_kv_to_fp16_prefix")


def kvq_bytes_per_token(fmt, heads, head_dim):
    """Bytes one token occupies in one cache tensor of a format (host only)."""
    rc = load_library().kvq_bytes_per_token(int(fmt), int(heads), int(head_dim))
    if rc < 0:
        raise KvqError(int(rc), "kvq_bytes_per_token")
    return int(rc)


# ---------------------------------------------------------------- host prefix compare
def kvq_count_match(a, b, max_a):
    """Length of the matching prefix of two 1-D host tensors / arrays of
    4- or 8-byte integers, at most max_a."""
    import numpy as np

    def host(x, name):
        if hasattr(x, "detach"):
            if x.device.type != "cpu":
                raise ValueError("%s must be in host memory" % name)
            x = x.detach().contiguous().numpy()
        x = np.ascontiguousarray(x)
        if x.ndim != 1:
            raise ValueError("%s must be 1-D" % name)
        return x

    a, b = host(a, "a"), host(b, "b")
    if a.dtype != b.dtype or a.itemsize not in (4, 8):
        raise TypeError("a and b must share a 4- or 8-byte integer dtype")
    rc = load_library().kvq_count_match(a.ctypes.data, a.size, b.ctypes.data, b.size,
                                        int(max_a), a.itemsize)
    if rc < 0:
        raise KvqError(int(rc), "kvq_count_match")
    return int(rc)


# ---------------------------------------------------------------- self-test hooks
def kvq_selftest_codes(x_bits, s_bits, wbits, out, force_clamp=False, stream=None):
    """out[i, j] = code of fp16 x_bits[j] under stored scale s_bits[i] (device
    16-bit tensors, out uint8 [ns, nx]).  force_clamp=False uses the kernels'
    own dispatch (defined for |x / s| < 2^(b-1) - 1/2 under normal scales)."""
    torch = _torch()
    dev = _device_of(x_bits)
    px = _dev_ptr(x_bits.view(torch.int16), "x", torch.int16)
    ps = _dev_ptr(s_bits.view(torch.int16), "s", torch.int16, dev)
    po = _dev_ptr(out, "out", torch.uint8, dev)
    _expect_shape(out, (s_bits.numel(), x_bits.numel()), "out")
    rc = load_library().kvq_selftest_codes(px, x_bits.numel(), ps, s_bits.numel(), int(wbits),
                                           int(bool(force_clamp)), po, _stream_handle(stream, dev))
    _check(rc, "kvq_selftest_codes")


def kvq_selftest_scales(a_bits, wbits, out, stream=None):
    """out[i] = stored fp16 scale of a block with absmax a_bits[i] (device
    16-bit tensors of the same shape)."""
    torch = _torch()
    dev = _device_of(a_bits)
    pa = _dev_ptr(a_bits.view(torch.int16), "absmax", torch.int16)
    po = _dev_ptr(out.view(torch.int16), "out", torch.int16, dev)
    _expect_shape(out, tuple(a_bits.shape), "out")
    rc = load_library().kvq_selftest_scales(pa, a_bits.numel(), int(wbits), po,
                                            _stream_handle(stream, dev))
    _check(rc, "kvq_selftest_scales")


def kvq_selftest_fastdiv(n, d, out, stream=None):
    """out[i] = n[i] // d through the kernels' multiply-shift divider (device
    int32 tensors, 0 <= n < 2^31, 1 <= d < 2^31)."""
    torch = _torch()
    dev = _device_of(n)
    pn = _dev_ptr(n, "n", torch.int32)
    po = _dev_ptr(out, "out", torch.int32, dev)
    _expect_shape(out, tuple(n.shape), "out")
    rc = load_library().kvq_selftest_fastdiv(pn, n.numel(), int(d), po, _stream_handle(stream, dev))
    _check(rc, "kvq_selftest_fastdiv")


def kvq_selftest_copy(src, dst, lane_bytes=16, group_waves=1, max_waves=0, stream=None):
    """dst = src through the library's plain non-temporal copy kernel (device
    uint8 tensors of equal size, a multiple of 16 bytes): the bandwidth
    reference of one launch."""
    torch = _torch()
    dev = _device_of(src)
    ps = _dev_ptr(src, "src", torch.uint8)
    pd = _dev_ptr(dst, "dst", torch.uint8, dev)
    _expect_shape(dst, tuple(src.shape), "dst")
    rc = load_library().kvq_selftest_copy(ps, pd, src.numel(), int(lane_bytes), int(group_waves),
                                          int(max_waves), _stream_handle(stream, dev))
    _check(rc, "kvq_selftest_copy")


def kvq_selftest_stream(src, dst, lane_elems=4, group_waves=1, stream=None):
    """Uneven-traffic bandwidth reference (device uint8 tensors): gather
    when src holds lane_elems times the bytes of dst (each 16-byte element
    of dst the XOR of lane_elems elements of src), scatter when dst holds
    lane_elems times the bytes of src (each element of src written
    lane_elems times)."""
    torch = _torch()
    dev = _device_of(src)
    ps = _dev_ptr(src, "src", torch.uint8)
    pd = _dev_ptr(dst, "dst", torch.uint8, dev)
    rc = load_library().kvq_selftest_stream(ps, src.numel(), pd, dst.numel(), int(lane_elems), int(group_waves),
                                            _stream_handle(stream, dev))
    _check(rc, "kvq_selftest_stream")
