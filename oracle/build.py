"""Build the CPU oracle (test infrastructure) into oracle/libkvq_oracle.so.

Plain gcc, IEEE arithmetic: no fast-math, no floating-point contraction.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "libkvq_oracle.so")
CFLAGS = ["-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(verbose=False):
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
