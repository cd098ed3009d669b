"""Build the gfx950 HIP library libkvq.so in-tree with hipcc.

Flags: IEEE arithmetic (no fast-math, no floating-point contraction), hidden
symbol visibility (only the KVQ_API entry points are exported), and packed
fp32 instructions disabled in device code.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = [os.path.join(CSRC, "kvq_kernels.hip"), os.path.join(CSRC, "kvq_api.cpp")]
HEADERS = [os.path.join(CSRC, "kvq_device.h"), os.path.join(CSRC, "kvq_internal.h"),
           os.path.join(ROOT, "include", "kvq.h"), os.path.join(ROOT, "include", "kvq_selftest.h")]
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-ffp-contract=off", "-fno-fast-math", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the kvq HIP library cannot be built")
    return path


def build(verbose=False):
    """Compile every source into kv_cache_quantization_kvq_amd/libkvq.so (always
    rebuilds)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, *HIPCC_FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "hip-link" not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
