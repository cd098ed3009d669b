"""The C ABI's host side (argument validation, extent and overlap
arithmetic at extreme sizes, count_match) built with g++ and the address and
undefined-behaviour sanitizers, aborting on the first report, and driven by
the host-side ABI tests in a Python process that preloads the address
sanitizer's runtime.  The kernel launchers are replaced by stand-ins that
return an error (tests/host_launch_stub.cpp); no test reaches them.  Then
20,000 random-argument calls of every entry point (tests/abi_fuzz.py) run
against the same build, and 5,000 calls that pass every check but the size
bound, with windows up to 2^28 rows: every call returns a documented code,
the sanitizers see no undefined behaviour in the validation arithmetic, and
no call the validation admits would launch more work-items than a dispatch's
32-bit grid size holds (the stand-in launchers check)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the host-side ABI tests that call into the library (not the ones that
# inspect the built HIP library's file or compile other programs)
HOST_TESTS = ("strerror_and_version or q_validation or selftest_fastdiv_validation or selftest_copy_validation or "
              "selftest_stream_validation or size_bounds or "
              "zero_work or fp8_validation or count_match or binding_host_checks or per_tensor_validation or "
              "prefix_validation or bytes_per_token")

DRIVER = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import kv_cache_quantization_kvq_amd as kvq
kvq._build.LIB = {lib!r}
kvq._LIB = None
import pytest
rc = pytest.main(["-q", "-s", "-p", "no:cacheprovider", {test_file!r}, "-k", {tests_k!r}])
if rc == 0:
    import abi_fuzz
    print("fuzz: %d random calls" % abi_fuzz.fuzz(kvq.load_library()), flush=True)
    print("fuzz: %d large valid calls reached a launcher" % abi_fuzz.fuzz_valid(kvq.load_library()), flush=True)
sys.exit(rc)
"""


def test_host_abi_under_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no C++ compiler")
    lib = str(tmp_path / "libkvq_host_sanitized.so")
    asan_rt = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan_rt) or not os.path.exists(asan_rt):
        pytest.skip("no address-sanitizer runtime")
    csrc = os.path.join(ROOT, "kv_cache_quantization_kvq_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fvisibility=hidden",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
                    "-I", os.path.join(ROOT, "include"), os.path.join(csrc, "kvq_api.cpp"),
                    os.path.join(ROOT, "tests", "host_launch_stub.cpp"), "-o", lib], check=True)
    driver = DRIVER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                           test_file=os.path.join(ROOT, "tests", "test_abi.py"), tests_k=HOST_TESTS)
    out = subprocess.run([sys.executable, "-c", driver], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, LD_PRELOAD=asan_rt, ASAN_OPTIONS="detect_leaks=0",
                                  UBSAN_OPTIONS="print_stacktrace=1"))
    assert out.returncode == 0, "exit %d\n%s\n%s" % (out.returncode, out.stdout[-3000:], out.stderr[-3000:])
    assert " passed" in out.stdout
    assert "fuzz: 20000 random calls" in out.stdout
    assert "large valid calls reached a launcher" in out.stdout
