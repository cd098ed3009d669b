"""Random-argument calls of every C-ABI entry point, for the host-only build
whose kernel launchers are stand-ins (tests/host_launch_stub.cpp).  Run by
tests/test_abi_sanitizers.py under the address and undefined-behaviour
sanitizers; never against the real library, because an accepted call with
a made-up device pointer would launch a kernel on it.

Each call must return success or one of the documented error codes (the
stand-in launchers make every accepted call return KVQ_ERR_HIP); any
out-of-range arithmetic in the validation is reported by the sanitizers.
count_match is called with real host arrays and consistent lengths only:
its contract makes the caller responsible for the lengths.
"""
import numpy as np

import kv_cache_quantization_kvq_amd as kvq

CODES = {0, -1, -2, -3, -4, -5, -6, -7}

I32 = [-(1 << 31), -7, -1, 0, 1, 2, 3, 7, 8, 31, 32, 33, 64, 96, 128, 255, 256, 1000, 4096, 65535, 65536,
       (1 << 20) - 1, 1 << 20, (1 << 20) + 1, (1 << 25), (1 << 30), (1 << 31) - 1]
FMT = [-1, 0, 1, 4, 5, 6, 8, 16]
BASE = 0x7F0000000000


def _int(rng):
    if rng.random() < 0.7:
        return int(rng.choice(I32))
    return int(rng.integers(-(1 << 31), 1 << 31))


def _small(rng):
    return int(rng.integers(-2, 40))


def _size(rng):
    return _int(rng) if rng.random() < 0.5 else _small(rng)


def _ptr(rng):
    r = rng.random()
    if r < 0.1:
        return None
    if r < 0.2:
        return BASE + int(rng.integers(1, 16))                    # misaligned
    return BASE + (int(rng.integers(0, 1 << 20)) << 32)           # aligned, far apart


def _shape(rng):
    return kvq.Shape(_size(rng), _size(rng), _size(rng), _size(rng))


def fuzz(lib, n=20000, seed=7):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        which = int(rng.integers(0, 12))
        if which == 0:
            rc = lib.kvq_fp16_to_fp8(_ptr(rng), _ptr(rng), _shape(rng), _size(rng), _size(rng), _size(rng), None)
        elif which == 1:
            rc = lib.kvq_fp8_to_fp16(_ptr(rng), _ptr(rng), _shape(rng), _size(rng), _size(rng), _size(rng), None)
        elif which in (2, 3):
            fn = lib.kvq_fp16_to_q_kv if which == 2 else lib.kvq_q_to_fp16_kv
            rc = fn(_ptr(rng), _ptr(rng), _ptr(rng), _ptr(rng), _ptr(rng), _ptr(rng), _shape(rng), _size(rng),
                    _size(rng), _size(rng), _size(rng), _ptr(rng), _ptr(rng), _size(rng), int(rng.choice(FMT)), None)
        elif which in (4, 5):
            fn = lib.kvq_fp16_to_kv if which == 4 else lib.kvq_kv_to_fp16
            rc = fn(_ptr(rng), _ptr(rng), _ptr(rng), int(rng.choice(FMT)), _ptr(rng), _ptr(rng), _ptr(rng),
                    int(rng.choice(FMT)), _shape(rng), _size(rng), _size(rng), _size(rng), _size(rng), _ptr(rng),
                    _ptr(rng), _size(rng), None)
        elif which == 6:
            rc = lib.kvq_kv_to_fp16_prefix(_ptr(rng), _ptr(rng), _ptr(rng), int(rng.choice(FMT)), _ptr(rng),
                                           _ptr(rng), _ptr(rng), int(rng.choice(FMT)), _shape(rng), _size(rng),
                                           _size(rng), _size(rng), _ptr(rng), _ptr(rng), _size(rng), None)
        elif which == 7:
            rc = lib.kvq_bytes_per_token(int(rng.choice(FMT)), _size(rng), _size(rng))
            assert rc >= 0 or rc in CODES, rc
            continue
        elif which == 10:
            size = _int(rng) * int(rng.choice([1, 16, 1024]))
            rc = lib.kvq_selftest_copy(_ptr(rng), _ptr(rng), size, int(rng.choice([0, 16, 32, 48, 64, 128, 256])),
                                       int(rng.choice([0, 1, 2, 3, 4, 8, 16])), _int(rng), None)
        elif which == 11:
            light = _int(rng) * int(rng.choice([1, 16, 1024]))
            k = int(rng.choice([1, 2, 3, 4, 8, 16]))
            heavy = light * k if rng.random() < 0.8 else _int(rng) * 1024
            src, dst = (heavy, light) if rng.random() < 0.5 else (light, heavy)
            rc = lib.kvq_selftest_stream(_ptr(rng), src, _ptr(rng), dst, int(rng.choice([0, 1, 2, 3, 4, 8, 16])),
                                         int(rng.choice([0, 1, 2, 4, 8, 16])), None)
        elif which == 8:
            f = lib.kvq_selftest_codes
            rc = f(_ptr(rng), _int(rng) * 8 if rng.random() < 0.5 else _int(rng), _ptr(rng), _int(rng),
                   int(rng.choice(FMT)), int(rng.integers(0, 2)), _ptr(rng), None)
        else:
            elem = int(rng.choice([4, 8]))
            la, lb = int(rng.integers(0, 50)), int(rng.integers(0, 50))
            a = rng.integers(0, 3, size=la).astype(np.int32 if elem == 4 else np.int64)
            b = rng.integers(0, 3, size=lb).astype(a.dtype)
            max_a = _int(rng)
            rc = lib.kvq_count_match(a.ctypes.data if la else None, la, b.ctypes.data if lb else None, lb,
                                     max_a, elem if rng.random() < 0.9 else int(rng.choice([0, 2, 16])))
            assert rc >= 0 or rc in CODES, rc
            continue
        assert rc in CODES, rc
    return n



def _far(k):
    return k << 42                    # buffers up to 4 TiB apart: no overlap below that size


def fuzz_valid(lib, n=5000, seed=8):
    """Calls that pass the shape, window, alignment and overlap checks, with
    windows up to 2^28 rows, so that the bound on a launch's size decides."""
    rng = np.random.default_rng(seed)
    accepted = 0
    for _ in range(n):
        which = int(rng.integers(0, 4))
        heads = int(rng.integers(1, 17))
        head_dim = 32 * int(rng.integers(1, 9))
        if which == 0:                                            # contiguous 8-bit
            dim0, dim1 = int(rng.integers(1, 5)), int(1 << int(rng.integers(0, 25)))
            shape = kvq.Shape(dim0, dim1, heads, head_dim)
            batch, width = int(rng.integers(1, dim0 + 1)), int(rng.integers(1, dim1 + 1))
            fn = lib.kvq_fp16_to_fp8 if rng.random() < 0.5 else lib.kvq_fp8_to_fp16
            rc = fn(_far(1), _far(2), shape, batch, 0, width, None)
        else:
            dim0, dim1 = int(1 << int(rng.integers(0, 15))), int(1 << int(rng.integers(0, 15)))
            shape = kvq.Shape(dim0, dim1, heads, head_dim)
            wb = int(rng.choice([4, 6, 8]))
            if which == 1:                                        # contiguous K/V
                batch, width = int(rng.integers(1, dim0 + 1)), int(rng.integers(1, dim1 + 1))
                fn = lib.kvq_fp16_to_q_kv if rng.random() < 0.5 else lib.kvq_q_to_fp16_kv
                rc = fn(_far(1), _far(2), _far(3), _far(4), _far(5), _far(6), shape, batch, 0, width, 0,
                        None, None, 0, wb, None)
            elif which == 2:                                      # paged K/V
                batch = int(1 << int(rng.integers(0, 15)))
                cols = max(1, (1 << 30) // dim1 // int(rng.integers(1, 4)))
                width = int(rng.integers(1, 1 << int(rng.integers(1, 29))))
                fn = lib.kvq_fp16_to_q_kv if rng.random() < 0.5 else lib.kvq_q_to_fp16_kv
                rc = fn(_far(1), _far(2), _far(3), _far(4), _far(5), _far(6), shape, batch, 0, width, dim1,
                        _far(7), _far(8), cols, wb, None)
            else:                                                 # full prefix
                batch = int(1 << int(rng.integers(0, 15)))
                cols = max(1, (1 << 30) // dim1 // int(rng.integers(1, 4)))
                max_len = int(rng.integers(1, 1 << int(rng.integers(1, 29))))
                rc = lib.kvq_kv_to_fp16_prefix(_far(1), _far(2), _far(3), wb, _far(4), _far(5), _far(6), wb,
                                               shape, batch, int(rng.integers(0, 300)), max_len, _far(7), _far(8),
                                               cols, None)
        assert rc in CODES, rc
        accepted += rc == -7
    return accepted
