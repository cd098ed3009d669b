"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every symbol its public headers declare, validates arguments before touching
the device, and computes count_match exactly.

Argument meanings follow the ExLlamaV2 cache page (Signature, I/O Contract):
batch_size, offset, width, page_size (0 = contiguous), cache_seqlens,
block_table, wbits in {4, 6}; count_match(a, b, max_a).
Fake device addresses are used only in calls that must be rejected by the
host validation (or do no work), so no kernel is ever launched here.

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_quantization_kvq_amd as kvq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

NULL, WBITS, SHAPE, RANGE, ALIGN, OVERLAP = -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.library_path()):
        kvq._build.build()
    return kvq.load_library()


def _declared_symbols():
    names = set()
    for h in ("kvq.h", "kvq_selftest.h"):
        with open(os.path.join(ROOT, "include", h)) as fh:
            text = fh.read()
        names |= set(re.findall(r"KVQ_API\s+[\w\s\*]+?\b(kvq_\w+)\s*\(", text))
    return names


def test_exports_every_declared_symbol(lib):
    names = _declared_symbols()
    assert {"kvq_fp16_to_fp8", "kvq_fp8_to_fp16", "kvq_fp16_to_q_kv", "kvq_q_to_fp16_kv",
            "kvq_count_match", "kvq_strerror", "kvq_selftest_codes"} <= names
    for n in names:
        assert hasattr(lib, n), n


def test_only_declared_symbols_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == _declared_symbols()


def test_c_consumer(tmp_path, lib):
    """A C99 program including the public headers, linked against the
    library, exercising the host-side entry points (no GPU call)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "c_abi_check"
    libdir = os.path.dirname(kvq.library_path())
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
           "-L", libdir, "-lkvq", "-Wl,-rpath," + libdir, "-o", str(exe)]
    subprocess.run(cmd, check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert "c abi ok" in out.stdout


def test_fastdiv_constants_on_host(tmp_path):
    """The host-computed multiply-shift constants of the row split give
    n / d exactly (integer division) for numerators below 2^31: every
    divisor up to 2^16, 2^k - 1 / 2^k / 2^k + 1 up to 2^31 - 1 and 2000
    random ones, at the edges of the first and last 64 multiples."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("no C++ compiler")
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "kv_cache_quantization_kvq_amd", "csrc"),
                    os.path.join(ROOT, "tests", "fastdiv_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "fastdiv ok" in out.stdout


def test_strerror_and_version(lib):
    assert kvq.kvq_strerror(0) == "success"
    for c in range(-7, 0):
        assert kvq.kvq_strerror(c) != "unknown error"
    assert kvq.kvq_strerror(-99) == "unknown error"
    assert kvq.kvq_version() >= 100


# ---------------------------------------------------------------- validation
A = 0x7F0000000000          # fake, 16-byte aligned device addresses (never dereferenced)
GB = 1 << 30


def shp(d0=4, d1=16, h=2, d=64):
    return kvq.Shape(d0, d1, h, d)


def q(lib, quant=True, k=(A, A + GB, A + 2 * GB), v=(A + 3 * GB, A + 4 * GB, A + 5 * GB),
      s=None, batch=2, offset=0, width=4, page_size=0, sl=None, bt=None, cols=0, wbits=4):
    fn = lib.kvq_fp16_to_q_kv if quant else lib.kvq_q_to_fp16_kv
    return fn(*k, *v, s or shp(), batch, offset, width, page_size, sl, bt, cols, wbits, None)


def test_q_validation(lib):
    assert q(lib, wbits=5) == WBITS
    assert q(lib, wbits=7) == WBITS
    assert q(lib, wbits=16) == WBITS
    assert q(lib, k=(A, None, A + 2 * GB)) == NULL                       # partial triple
    assert q(lib, k=(None, None, None), v=(None, None, None)) == NULL
    assert q(lib, s=shp(d=48)) == SHAPE                                    # head_dim % 32
    assert q(lib, s=shp(h=0)) == SHAPE
    assert q(lib, batch=5) == RANGE                                        # > dim0
    assert q(lib, offset=13, width=4) == RANGE                             # past dim1
    assert q(lib, batch=-1) == RANGE
    assert q(lib, k=(A + 8, A + GB, A + 2 * GB)) == ALIGN
    assert q(lib, k=(A, A, A + 2 * GB)) == OVERLAP                         # in == out
    assert q(lib, k=(A, A + GB, A + 2 * GB), v=(A + 3 * GB, A + GB + 64, A + 5 * GB)) == OVERLAP
    # paged: page_size must equal dim1, tables required, columns positive
    assert q(lib, page_size=8, sl=A + 6 * GB, bt=A + 7 * GB, cols=4) == SHAPE
    assert q(lib, page_size=16, sl=None, bt=A + 7 * GB, cols=4) == NULL
    assert q(lib, page_size=16, sl=A + 6 * GB, bt=A + 7 * GB, cols=0) == RANGE
    assert q(lib, page_size=16, sl=A + 6 * GB + 2, bt=A + 7 * GB, cols=4) == ALIGN
    assert q(lib, page_size=-1) == RANGE
    # dequant validates the same way
    assert q(lib, quant=False, wbits=3) == WBITS
    assert q(lib, quant=False, k=(A, A, A + 2 * GB)) == OVERLAP


def test_selftest_fastdiv_validation(lib):
    f = lib.kvq_selftest_fastdiv
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    assert f(A, 16, 0, A + GB, None) == RANGE
    assert f(A, 16, 1 << 31, A + GB, None) == RANGE
    assert f(A, -1, 7, A + GB, None) == RANGE
    assert f(None, 16, 7, A + GB, None) == NULL
    assert f(A + 2, 16, 7, A + GB, None) == ALIGN
    assert f(A, 0, 7, A + GB, None) == 0


def test_selftest_copy_validation(lib):
    """The bandwidth-reference copy rejects every bad argument before any
    launch; zero bytes return without one."""
    f = lib.kvq_selftest_copy
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_void_p]
    assert f(None, A + GB, 1024, 16, 1, 0, None) == NULL
    assert f(A, None, 1024, 16, 1, 0, None) == NULL
    assert f(A, A + GB, -16, 16, 1, 0, None) == RANGE
    assert f(A, A + GB, 1000, 16, 1, 0, None) == RANGE          # not a multiple of 16
    assert f(A, A + GB, 1024, 16, 1, -1, None) == RANGE
    for lb in (0, 8, 48, 256):
        assert f(A, A + GB, 1024, lb, 1, 0, None) == RANGE
    for gw in (0, 3, 16):
        assert f(A, A + GB, 1024, 16, gw, 0, None) == RANGE
    assert f(A + 8, A + GB, 1024, 16, 1, 0, None) == ALIGN
    assert f(A, A + GB + 4, 1024, 16, 1, 0, None) == ALIGN
    assert f(A, A + 512, 1024, 16, 1, 0, None) == OVERLAP
    assert f(A, A, 1024, 16, 1, 0, None) == OVERLAP
    assert f(A, A + GB, 0, 16, 1, 0, None) == 0


def test_selftest_stream_validation(lib):
    """The uneven-traffic reference accepts only the two size ratios, whole
    1024-byte tiles on the light side and the listed lane and group sizes,
    and rejects everything else before any launch; zero sizes return
    without one."""
    f = lib.kvq_selftest_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    assert f(None, 4096, A + GB, 1024, 4, 1, None) == NULL
    assert f(A, 4096, None, 1024, 4, 1, None) == NULL
    for le in (0, 1, 3, 16):
        assert f(A, 4096 * le, A + GB, 4096, le, 1, None) == RANGE
    for gw in (0, 3, 16):
        assert f(A, 4096, A + GB, 1024, 4, gw, None) == RANGE
    assert f(A, 4096, A + GB, 2048, 4, 1, None) == RANGE          # neither ratio
    assert f(A, 2048, A + GB, 512, 4, 1, None) == RANGE           # light side not whole tiles
    assert f(A, -4096, A + GB, -1024, 4, 1, None) == RANGE
    assert f(A, 1 << 56, A + GB, 1 << 54, 4, 1, None) == RANGE
    assert f(A + 8, 4096, A + GB, 1024, 4, 1, None) == ALIGN
    assert f(A, 4096, A + 2048, 1024, 4, 1, None) == OVERLAP       # gather
    assert f(A, 1024, A + 512, 4096, 4, 1, None) == OVERLAP        # scatter
    assert f(A, 0, A + GB, 0, 4, 1, None) == 0


def test_size_bounds(lib):
    """Rows up to 2^20 elements are accepted, longer ones are SHAPE; a call
    whose work units exceed the 32-bit numbering is RANGE (checked before any
    launch: batch 0 returns without one)."""
    assert q(lib, s=shp(d0=1, d1=2, h=8192, d=128), batch=0, width=2) == 0
    assert q(lib, s=shp(d0=1, d1=2, h=8193, d=128), batch=0, width=2) == SHAPE
    assert q(lib, s=shp(d0=1 << 16, d1=1 << 15, h=8, d=128), batch=1 << 16, width=1 << 15) == RANGE
    assert q(lib, s=shp(d0=1 << 16, d1=1 << 15, h=8, d=128), batch=1 << 16, width=1 << 15,
             quant=False) == RANGE
    f = lib.kvq_fp16_to_fp8
    assert f(A, A + GB, shp(d0=1, d1=2, h=8193, d=128), 0, 0, 2, None) == SHAPE
    # a launch's work-items must fit 32 bits: batch * width * 2 tensors *
    # ceil(R / 512) segments is at most 2^26 - 64 (R = 1024: 2 per row)
    far3 = ((1 << 60), (2 << 60), (3 << 60))
    far6 = ((4 << 60), (5 << 60), (6 << 60))
    s_big = shp(d0=1 << 13, d1=1 << 12, h=8, d=128)
    assert q(lib, s=s_big, k=far3, v=far6, batch=1 << 13, width=1 << 11) == RANGE     # 2^26
    assert q(lib, s=s_big, k=far3, v=far6, batch=1 << 13, width=(1 << 11) - 1) != RANGE
    assert f(1 << 60, 2 << 60, shp(d0=1, d1=1 << 25, h=8, d=128), 1, 0, 1 << 25, None) == RANGE
    assert f(1 << 60, 2 << 60, shp(d0=1, d1=1 << 25, h=8, d=128), 1, 0, (1 << 25) - 8, None) != RANGE
    # a cache beyond 2^60 elements is RANGE, whatever the window
    big = shp(d0=(1 << 31) - 1, d1=(1 << 31) - 1, h=8, d=128)
    assert q(lib, s=big, batch=0) == RANGE
    assert f(A, A + GB, big, 0, 0, 2, None) == RANGE
    far = (1 << 60, 2 << 60, 3 << 60)                      # 2^50 elements: 2 PiB of fp16
    assert q(lib, s=shp(d0=1 << 20, d1=1 << 20, h=8, d=128), k=far, v=(None,) * 3, batch=0) == 0
    # extreme table extents of a call with nothing to do: no overflow, success;
    # a table row addresses at most 2^30 positions (cols * page_size)
    assert q(lib, s=shp(d0=4, d1=1), page_size=1, sl=A + 6 * GB, bt=A + 7 * GB, cols=1 << 30,
             batch=(1 << 31) - 1, width=0) == 0
    assert q(lib, s=shp(d0=4, d1=1), page_size=1, sl=A + 6 * GB, bt=A + 7 * GB, cols=(1 << 30) + 1,
             batch=1, width=0) == RANGE
    assert q(lib, s=shp(d0=4, d1=2), page_size=2, sl=A + 6 * GB, bt=A + 7 * GB, cols=1 << 29,
             batch=1, width=0) == 0
    assert q(lib, s=shp(d0=4, d1=2), page_size=2, sl=A + 6 * GB, bt=A + 7 * GB, cols=(1 << 29) + 1,
             batch=1, width=0) == RANGE


def test_q_zero_work_returns_ok(lib):
    # valid arguments but nothing to do: no launch, success
    assert q(lib, width=0) == 0
    assert q(lib, batch=0) == 0
    assert q(lib, width=0, wbits=8) == 0 and q(lib, quant=False, width=0, wbits=6) == 0
    assert q(lib, k=(None, None, None), width=0) == 0
    assert q(lib, page_size=16, sl=A + 6 * GB, bt=A + 7 * GB, cols=4, batch=0) == 0
    # paged mode allows batch_size > dim0 (sequences are not pages)
    assert q(lib, page_size=16, sl=A + 6 * GB, bt=A + 7 * GB, cols=4, batch=9, width=0) == 0


def test_fp8_validation(lib):
    f = lib.kvq_fp16_to_fp8
    assert f(None, A + GB, shp(), 1, 0, 4, None) == NULL
    assert f(A, A + GB, kvq.Shape(2, 8, 3, 5), 1, 0, 4, None) == SHAPE    # R = 15
    assert f(A, A + GB, shp(), 5, 0, 4, None) == RANGE
    assert f(A, A + GB, shp(), 1, -1, 4, None) == RANGE
    assert f(A, A + 4, shp(), 1, 0, 4, None) == ALIGN
    assert f(A, A + 96, shp(), 1, 0, 4, None) == OVERLAP                  # inside the fp16 input
    assert f(A, A + GB, shp(), 1, 0, 0, None) == 0
    assert lib.kvq_fp8_to_fp16(A, A + 64, shp(), 1, 0, 4, None) == OVERLAP
    assert lib.kvq_fp8_to_fp16(A, A + GB, kvq.Shape(2, 8, 3, 8), 0, 0, 4, None) == 0   # R = 24


# ---------------------------------------------------------------- count_match
def _cm(lib, a, b, max_a):
    return lib.kvq_count_match(a.ctypes.data, a.size, b.ctypes.data, b.size, max_a, a.itemsize)


def test_count_match_errors(lib):
    a = np.zeros(4, np.int32)
    assert lib.kvq_count_match(a.ctypes.data, 4, a.ctypes.data, 4, 4, 2) == RANGE
    assert lib.kvq_count_match(a.ctypes.data, -1, a.ctypes.data, 4, 4, 4) == RANGE
    assert lib.kvq_count_match(None, 4, a.ctypes.data, 4, 4, 4) == NULL
    assert lib.kvq_count_match(None, 0, None, 0, 4, 4) == 0


@pytest.mark.parametrize("dtype", [np.int32, np.int64])
def test_count_match_bruteforce(lib, dtype):
    """Every length 0..40, every planted mismatch position, several caps and
    base offsets that break 8-byte alignment, against the oracle's loop."""
    rng = np.random.default_rng(71)
    buf_a = np.zeros(64, dtype)
    buf_b = np.zeros(64, dtype)
    for n in range(0, 41):
        for start in (0, 1, 3):
            a = buf_a[start:start + n]
            b = buf_b[start:start + n]
            a[:] = rng.integers(0, 1 << 17, size=n)
            for m in list(range(n + 1)):
                b[:] = a
                if m < n:
                    b[m] = a[m] ^ 1
                for max_a in (n, n + 5, m, max(m - 1, 0), -2):
                    want = oracle.count_match(a, b, max_a)
                    assert want == min(m, max(max_a, 0))
                    assert _cm(lib, a, b, max_a) == want


@pytest.mark.parametrize("dtype", [np.int32, np.int64])
def test_count_match_exact_buffers(lib, dtype):
    """Each array in an allocation of exactly its own length (no slack after
    the last element, so a read past it is out of bounds), every length
    0..40, equal and with the last element differing."""
    rng = np.random.default_rng(72)
    for n in range(0, 41):
        a = rng.integers(0, 1 << 17, size=n).astype(dtype)
        b = a.copy()
        assert _cm(lib, a, b, n) == n
        if n:
            b[-1] ^= 1
            assert _cm(lib, a, b, n) == n - 1


def test_count_match_long_planted(lib):
    w = __import__("kv_cache_quantization_kvq_amd.synth", fromlist=["x"])
    rng = np.random.default_rng(1005)
    for _ in range(20):
        a, b, m = w.token_ids(rng, 65536)
        assert kvq.kvq_count_match(a, b, 65536) == m
        assert kvq.kvq_count_match(a, b, 1000) == min(m, 1000)
        assert oracle.count_match(a, b, 65536) == m


def test_count_match_torch_inputs():
    import torch
    a = torch.arange(100, dtype=torch.int64)
    b = a.clone()
    b[37] = -1
    assert kvq.kvq_count_match(a, b, 1000) == 37
    with pytest.raises(TypeError):
        kvq.kvq_count_match(a, b.to(torch.int32), 10)


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built HIP library every entry point raises: there is no
    fallback path."""
    monkeypatch.setattr(kvq, "_LIB", None)
    monkeypatch.setattr(kvq._build, "LIB", "/nonexistent/libkvq.so")
    with pytest.raises(RuntimeError):
        kvq.load_library()
    with pytest.raises(RuntimeError):
        kvq.kvq_version()
    with pytest.raises(RuntimeError):
        kvq.kvq_count_match(np.arange(4, dtype=np.int32), np.arange(4, dtype=np.int32), 4)


def test_binding_host_checks():
    """The Python binding checks dtypes, devices and arguments before it calls
    the library (host tensors are rejected: the library takes device
    pointers)."""
    import torch
    shape = (2, 4, 2, 64)
    f16 = torch.zeros(shape, dtype=torch.float16)
    f32 = torch.zeros(shape, dtype=torch.float32)
    codes = torch.zeros(kvq.code_shape(shape, 4), dtype=torch.uint8)
    scales = torch.zeros(kvq.scale_shape(shape), dtype=torch.float16)
    with pytest.raises(TypeError):
        kvq.kvq_fp16_to_q_kv(f32, codes, scales, None, None, None, 1, 0, 2)
    with pytest.raises(ValueError):
        kvq.kvq_fp16_to_q_kv(f16, codes, scales, None, None, None, 1, 0, 2)      # host memory
    with pytest.raises(TypeError):
        kvq.kvq_fp16_to_fp8(f32, torch.zeros(shape, dtype=torch.uint8), 1, 0, 2)
    with pytest.raises(ValueError):
        kvq.kvq_fp16_to_kv(None, None, None, 4, None, None, None, 4, 1, 0, 2)     # neither K nor V
    with pytest.raises(ValueError):
        kvq.kvq_fp16_to_kv(f16, codes, scales, 5, None, None, None, 4, 1, 0, 2)   # unknown format
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_bytes_per_token(5, 8, 128)
    assert e.value.code == WBITS
    assert kvq.compact_shape(shape, kvq.KVQ_FMT_FP8) == shape
    assert kvq.compact_shape(shape, kvq.KVQ_FMT_Q6) == (2, 4, 2, 48)


# ---------------------------------------------------------------- per-tensor formats, prefix, capacity
def kv(lib, to_compact=True, k=(A, A + GB, A + 2 * GB), fk=4, v=(A + 3 * GB, A + 4 * GB, A + 5 * GB), fv=4,
       s=None, batch=2, offset=0, width=4, page_size=0, sl=None, bt=None, cols=0):
    fn = lib.kvq_fp16_to_kv if to_compact else lib.kvq_kv_to_fp16
    return fn(k[0], k[1], k[2], fk, v[0], v[1], v[2], fv, s or shp(), batch, offset, width, page_size,
              sl, bt, cols, None)


def test_per_tensor_validation(lib):
    assert kv(lib, fk=5) == WBITS
    assert kv(lib, fv=16) == WBITS
    assert kv(lib, fk=0) == NULL                                     # 8-bit with a scales pointer
    assert kv(lib, fk=0, k=(A, A + GB, None), width=0) == 0          # 8-bit without scales: fine
    assert kv(lib, fk=4, k=(A, A + GB, None)) == NULL                # block format needs scales
    assert kv(lib, k=(A, None, None)) == NULL                        # partial
    assert kv(lib, k=(None, None, A + 2 * GB)) == NULL               # scales of an absent tensor
    assert kv(lib, k=(None, None, None), v=(None, None, None)) == NULL
    assert kv(lib, k=(None, None, None), fk=99, width=0) == 0         # absent tensor: format ignored
    assert kv(lib, s=shp(d=48)) == SHAPE
    assert kv(lib, batch=5) == RANGE
    assert kv(lib, k=(A, A, A + 2 * GB)) == OVERLAP
    assert kv(lib, to_compact=False, fk=0, k=(A, A + GB, None), fv=6, width=0) == 0
    assert kv(lib, page_size=16, sl=A + 6 * GB, bt=A + 7 * GB, cols=0) == RANGE
    assert kv(lib, page_size=16, sl=A + 6 * GB, bt=A + 7 * GB, cols=4, width=0) == 0


def test_prefix_validation(lib):
    f = lib.kvq_kv_to_fp16_prefix

    def call(k=(A, A + GB, A + 2 * GB), fk=4, batch=2, width=1, max_len=64, sl=A + 6 * GB, bt=A + 7 * GB, cols=4, s=None):
        return f(k[0], k[1], k[2], fk, None, None, None, 0, s or shp(), batch, width, max_len, sl, bt, cols, None)

    assert call(max_len=-1) == RANGE
    assert call(cols=0) == RANGE
    assert call(width=-1) == RANGE
    assert call(sl=None) == NULL
    assert call(fk=3) == WBITS
    assert call(s=shp(d=40)) == SHAPE
    assert call(max_len=0) == 0
    assert call(batch=0) == 0


def test_bytes_per_token_closed_form(lib):
    for heads, head_dim in ((8, 128), (32, 128), (1, 32), (4, 64)):
        R = heads * head_dim
        assert kvq.kvq_bytes_per_token(kvq.KVQ_FMT_FP16, heads, head_dim) == 2 * R
        assert kvq.kvq_bytes_per_token(kvq.KVQ_FMT_FP8, heads, head_dim) == R
        assert kvq.kvq_bytes_per_token(kvq.KVQ_FMT_Q4, heads, head_dim) == R // 2 + R // 16
        assert kvq.kvq_bytes_per_token(kvq.KVQ_FMT_Q6, heads, head_dim) == 3 * R // 4 + R // 16
        assert kvq.kvq_bytes_per_token(kvq.KVQ_FMT_Q8, heads, head_dim) == R + R // 16
        for fmt in (0, 4, 6, 8, 16):
            assert kvq.kvq_bytes_per_token(fmt, heads, head_dim) == oracle.bytes_per_token(fmt, heads, head_dim)
    assert lib.kvq_bytes_per_token(5, 8, 128) == WBITS
    assert lib.kvq_bytes_per_token(4, 8, 48) == SHAPE
    assert lib.kvq_bytes_per_token(16, 0, 128) == SHAPE


def test_one_hip_runtime_whatever_the_import_order():
    """torch ships its own HIP runtime.  The binding loads libkvq.so only after
    torch, so a program that loads the library before it imports torch still
    holds one HIP runtime and one HSA runtime, the ones its tensors and
    streams come from."""
    import subprocess
    import sys
    code = "\n".join([
        "import sys",
        "sys.path.insert(0, %r)" % ROOT,
        "import kv_cache_quantization_kvq_amd as kvq",
        "kvq.load_library()",
        "import torch",
        "maps = open('/proc/self/maps').read().splitlines()",
        "for lib in ('libamdhip64', 'libhsa-runtime64'):",
        "    print(lib, len({l.split()[-1] for l in maps if lib in l}))",
    ])
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert "libamdhip64 1" in out.stdout and "libhsa-runtime64 1" in out.stdout, out.stdout
