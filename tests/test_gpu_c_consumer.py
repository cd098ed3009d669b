"""A plain C program drives the GPU conversions through include/kvq.h, with
device memory and a stream from the HIP runtime's C API (no Python binding,
no torch), and compares every output byte with the oracle's C functions:
paged Q4 / Q6 / Q8 round trips with invalid table entries and a partial row
segment, and contiguous 8-bit both ways.  (Operations: ExLlamaV2 cache page,
Signature / I/O Contract; the boundary is the C ABI of include/kvq.h.)

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import os
import shutil
import subprocess
import sys

import pytest

import kv_cache_quantization_kvq_amd as kvq
import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_program_through_the_abi(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    lib_dir = os.path.dirname(kvq.library_path())
    assert os.path.exists(kvq.library_path()), "libkvq.so is not built"
    oracle.lib()                                        # builds the oracle library if absent
    oracle_dir = os.path.join(ROOT, "oracle")
    assert os.path.exists(os.path.join(oracle_dir, "libkvq_oracle.so"))
    exe = tmp_path / "c_gpu_consumer"
    cmd = ["gcc", "-std=gnu11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_gpu_consumer.c"),
           "-L", lib_dir, "-lkvq", "-L", oracle_dir, "-lkvq_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + oracle_dir, "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True)
    print("running the C consumer", flush=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=90)
    assert out.returncode == 0, "exit %d: %s" % (out.returncode, out.stderr)
    assert "c gpu consumer ok" in out.stdout


def test_library_loaded_before_torch():
    """A Python program that loads the library before it imports torch (torch
    ships its own HIP runtime): a paged Q4 round trip and a full-prefix widen
    still match the oracle byte for byte."""
    code = "\n".join([
        "import sys",
        "sys.path.insert(0, %r)" % ROOT,
        "import numpy as np",
        "import kv_cache_quantization_kvq_amd as kvq",
        "import oracle",
        "kvq.load_library()",
        "import torch",
        "rng = np.random.default_rng(11)",
        "shape = (8, 4, 2, 64)",
        "k = rng.standard_normal(shape).astype(np.float16)",
        "v = rng.standard_normal(shape).astype(np.float16)",
        "bt = rng.permutation(8).astype(np.int32)[:6].reshape(2, 3)",
        "sl = np.array([1, 5], np.int32)",
        "d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()",
        "cs, ss = kvq.code_shape(shape, 4), kvq.scale_shape(shape)",
        "kq, vq = torch.zeros(cs, dtype=torch.uint8, device='cuda'), torch.zeros(cs, dtype=torch.uint8, device='cuda')",
        "ks, vs = torch.zeros(ss, dtype=torch.float16, device='cuda'), torch.zeros(ss, dtype=torch.float16, device='cuda')",
        "ko, vo = torch.zeros(shape, dtype=torch.float16, device='cuda'), torch.zeros(shape, dtype=torch.float16, device='cuda')",
        "pk, pv = torch.zeros(shape, dtype=torch.float16, device='cuda'), torch.zeros(shape, dtype=torch.float16, device='cuda')",
        "a = (2, 0, 6, 4, d(sl), d(bt))",
        "kvq.kvq_fp16_to_q_kv(d(k), kq, ks, d(v), vq, vs, *a, wbits=4)",
        "kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, *a, wbits=4)",
        "kvq.kvq_kv_to_fp16_prefix(kq, pk, ks, 4, vq, pv, vs, 4, 2, 6, 12, d(sl), d(bt))",
        "torch.cuda.synchronize()",
        "okq, ovq = np.zeros(cs, np.uint8), np.zeros(cs, np.uint8)",
        "oks, ovs = np.zeros(ss, np.float16), np.zeros(ss, np.float16)",
        "oko, ovo = np.zeros(shape, np.float16), np.zeros(shape, np.float16)",
        "opk, opv = np.zeros(shape, np.float16), np.zeros(shape, np.float16)",
        "oracle.fp16_to_q_kv(k, okq, oks, v, ovq, ovs, 2, 0, 6, 4, sl, bt, 4)",
        "oracle.q_to_fp16_kv(okq, oko, oks, ovq, ovo, ovs, 2, 0, 6, 4, sl, bt, 4)",
        "oracle.kv_to_fp16_prefix(okq, opk, oks, 4, ovq, opv, ovs, 4, 2, 6, 12, sl, bt)",
        "pairs = ((kq, okq), (vq, ovq), (ks, oks), (vs, ovs), (ko, oko), (vo, ovo), (pk, opk), (pv, opv))",
        "assert all(np.array_equal(g.cpu().numpy().view(np.uint8), w.view(np.uint8)) for g, w in pairs)",
        "print('library-first ok', flush=True)",
    ])
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, "exit %d: %s" % (out.returncode, out.stderr[-3000:])
    assert "library-first ok" in out.stdout
