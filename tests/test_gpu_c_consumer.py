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
