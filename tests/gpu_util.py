"""Helpers shared by the GPU tests: device buffers, sentinels, row gathers.
Pure plumbing (allocation, copies, indexing); no conversion arithmetic."""
import numpy as np

SENTINEL = 0xA5


def torch():
    import torch as _t
    return _t


def need_lib():
    import kv_cache_quantization_kvq_amd as kvq
    kvq.load_library()          # raises if the HIP library is missing
    return kvq


def dev(arr):
    """Host numpy array -> device tensor (fp16 stays fp16, uint16 bits -> fp16)."""
    t = torch()
    if arr.dtype == np.uint16:
        arr = arr.view(np.float16)
    return t.from_numpy(np.ascontiguousarray(arr)).cuda()


def host(t):
    """Device tensor -> host numpy (fp16 returned as uint16 bits)."""
    torch().cuda.synchronize()
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.float16 else a


def sentinel(shape, dtype):
    t = torch()
    out = t.empty(shape, dtype=dtype, device="cuda")
    out.view(t.uint8).fill_(SENTINEL)
    return out


def sentinel_np(shape, dtype):
    a = np.empty(shape, dtype)
    a.view(np.uint8)[...] = SENTINEL
    return a


def rows_view(t):
    """[dim0, dim1, heads, x] -> [dim0 * dim1, heads * x] view."""
    return t.view(t.shape[0] * t.shape[1], -1)


def gather_rows(t, rows):
    """Rows (flat indices into dim0 * dim1) of a device cache, to host."""
    tt = torch()
    idx = tt.from_numpy(np.asarray(rows, np.int64)).cuda()
    return host(rows_view(t).index_select(0, idx))


def byte_diff(a, b, what):
    a = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    b = np.ascontiguousarray(b).view(np.uint8).reshape(-1)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    bad = np.nonzero(a != b)[0]
    if bad.size:
        raise AssertionError("%s: %d of %d bytes differ, first at byte %d (gpu %#x vs oracle %#x)"
                             % (what, bad.size, a.size, bad[0], a[bad[0]], b[bad[0]]))
