"""Planted mistakes in the oracle must fail its pins.

Each mutant below is a copy of oracle/kvq_oracle.c with one plausible
mistake planted (a wrong divisor, rounding rule, clamp bound, offset, bit
order, dropped term, swapped operand, off-by-one), built with the oracle's
own flags.  The oracle pin suites (test_oracle_codec.py, test_oracle_quant.py,
test_oracle_layout.py) are then run against that build, in a subprocess that
loads it through KVQ_ORACLE_LIB, and must fail.  The unmodified source, built
the same way, must pass them.  This checks that the pins are anchored to the
pages' definitions and to mathematics rather than to the oracle itself: a
mistake anywhere in it is caught.  The mistakes are all memory-safe (every
index stays inside the buffers the tests allocate), so a mutant fails by an
assertion, not a crash.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle.build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# run order: the quicker suites first (each mutant stops at its first failure)
PIN_FILES = ["tests/test_oracle_layout.py", "tests/test_oracle_codec.py", "tests/test_oracle_quant.py"]

# (what the mistake is, [(text in kvq_oracle.c, replacement, occurrences)])
MUTANTS = [
    ("scale divides by 2^(b-1) instead of 2^(b-1) - 1",
     [("static int qmax_of(int wbits) { return (1 << (wbits - 1)) - 1; }",
       "static int qmax_of(int wbits) { return 1 << (wbits - 1); }", 1)]),
    ("codes round half away from zero",
     [("float r = nearbyintf(v);", "float r = roundf(v);", 1)]),
    ("lower clamp bound 1 - Z instead of -Z",
     [("if (r < (float)(-Z)) r = (float)(-Z);", "if (r < (float)(1 - Z)) r = (float)(1 - Z);", 1)]),
    ("upper clamp bound Z instead of Z - 1",
     [("if (r > (float)(Z - 1)) r = (float)(Z - 1);", "if (r > (float)Z) r = (float)Z;", 1)]),
    ("zero scale stores code -Z instead of 0",
     [("            q = 0;\n", "            q = -Z;\n", 1)]),
    ("two's complement storage instead of offset binary",
     [("u[i] = (uint8_t)(q + Z);", "u[i] = (uint8_t)(q & ((1 << wbits) - 1));", 1)]),
    ("absmax on signed values",
     [("double m = fabs(orc_f16_decode(x[i]));", "double m = orc_f16_decode(x[i]);", 1)]),
    ("absmax over half of the block",
     [("for (int i = 0; i < L; ++i) {\n        double m", "for (int i = 0; i < L / 2; ++i) {\n        double m", 1)]),
    ("dequantize subtracts Z - 1",
     [("int q = (int)u[i] - Z;", "int q = (int)u[i] - (Z - 1);", 1)]),
    ("fp16 rounding truncates above the half",
     [("if (frac > 0.5) return fl + 1.0;", "if (frac > 0.5) return fl;", 1)]),
    ("fp16 ties round up instead of to even",
     [("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;", 1)]),
    ("fp16 overflow threshold at 65504",
     [("if (a >= 65520.0) return", "if (a >= 65504.0) return", 1)]),
    ("fp16 subnormal quantum 2^-23",
     [("v = ldexp((double)m, -24);", "v = ldexp((double)m, -23);", 1)]),
    ("bits of each byte packed most significant first (pack and unpack agree)",
     [("out[bit / 8] |= (uint8_t)(1u << (bit % 8));", "out[bit / 8] |= (uint8_t)(0x80u >> (bit % 8));", 1),
      ("if ((in[bit / 8] >> (bit % 8)) & 1)", "if ((in[bit / 8] >> (7 - bit % 8)) & 1)", 1)]),
    ("each code's bits stored most significant first (pack and unpack agree)",
     [("if ((u[j] >> k) & 1)", "if ((u[j] >> (wbits - 1 - k)) & 1)", 1),
      ("v |= 1 << k;", "v |= 1 << (wbits - 1 - k);", 1)]),
    ("8-bit narrowing keeps bits 7..14",
     [("return (uint8_t)(h >> 8); }", "return (uint8_t)(h >> 7); }", 1)]),
    ("8-bit widening fills the low byte with 0x80",
     [("return (uint16_t)((uint16_t)b << 8); }", "return (uint16_t)(((uint16_t)b << 8) | 0x80); }", 1)]),
    ("8-bit windows ignore the offset",
     [("int64_t row = (int64_t)b * dim1 + offset + t;", "int64_t row = (int64_t)b * dim1 + t;", 2)]),
    ("contiguous rows ignore the window offset",
     [("return (int64_t)b * dim1 + offset + t;", "return (int64_t)b * dim1 + t;", 1)]),
    ("paged positions ignore the offset",
     [("int64_t p = (int64_t)cache_seqlens[b] + offset + t;", "int64_t p = (int64_t)cache_seqlens[b] + t;", 1)]),
    ("the last physical page is treated as invalid",
     [("if (page < 0 || page >= dim0) return -1;", "if (page < 0 || page >= dim0 - 1) return -1;", 2)]),
    ("slot taken from the page index instead of the position",
     [("return page * page_size + p % page_size;", "return page * page_size + pi % page_size;", 2)]),
    ("K dequantized with V's scales",
     [("orc_dequant_rows(k_in + row * cb, k_scales + row * sb, 1, R, wbits, k_out + row * R);",
       "orc_dequant_rows(k_in + row * cb, (v_scales ? v_scales : k_scales) + row * sb, 1, R, wbits, k_out + row * R);",
       1)]),
    ("full prefix ends at cache_seqlens without the new tokens",
     [("int64_t end = (int64_t)cache_seqlens[b] + width;", "int64_t end = (int64_t)cache_seqlens[b];", 2)]),
    ("full prefix clipped one position short of max_len",
     [("if (end > max_len) end = max_len;", "if (end > max_len) end = max_len - 1;", 2)]),
    ("count_match compares only the first byte of each element",
     [("(size_t)elem_bytes) != 0)", "(size_t)1) != 0)", 1)]),
    ("count_match returns one past the first mismatch",
     [("            return i;\n", "            return i + 1;\n", 1)]),
    ("count_match ignores max_a",
     [("int64_t n = max_a;", "int64_t n = len_a;", 1)]),
    ("negative positions taken as position 0 instead of skipped",
     [("if (p < 0) return -1;", "if (p < 0) p = 0;", 1)]),
    ("codes multiply by a rounded reciprocal of the scale",
     [("float v = xf / sf;", "float v = xf * (1.0f / sf);", 1)]),
    ("codes not clamped",
     [("            if (r < (float)(-Z)) r = (float)(-Z);\n", "", 1),
      ("            if (r > (float)(Z - 1)) r = (float)(Z - 1);\n", "", 1)]),
    ("pieces of a long row packed at the row start (pack and unpack agree)",
     [("orc_pack_bits(u, len, wbits, crow + (int64_t)base * wbits / 8);", "orc_pack_bits(u, len, wbits, crow);", 1),
      ("orc_unpack_bits(crow + (int64_t)base * wbits / 8, len, wbits, u);", "orc_unpack_bits(crow, len, wbits, u);", 1)]),
    ("8-bit narrowing rounds to nearest instead of truncating",
     [("{ return (uint8_t)(h >> 8); }", "{ return (uint8_t)((h + 0x80u) >> 8); }", 1)]),
    ("bytes per token without the scales",
     [("return orc_fmt_row_bytes(R, fmt) + 2 * orc_fmt_scale_count(R, fmt);",
       "return orc_fmt_row_bytes(R, fmt);", 1)]),
]


def _source():
    with open(oracle_build.SRC) as fh:
        return fh.read()


def _build(text, out_dir, name):
    src = os.path.join(out_dir, name + ".c")
    lib = os.path.join(out_dir, name + ".so")
    with open(src, "w") as fh:
        fh.write(text)
    subprocess.run(["gcc", *oracle_build.CFLAGS, src, "-o", lib, "-lm"], check=True,
                   capture_output=True, text=True)
    return lib


def _run_pins(lib, stop_at_first):
    env = dict(os.environ, KVQ_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *PIN_FILES]
    if stop_at_first:
        cmd.insert(3, "-x")
    out = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return out.returncode, out.stdout[-2000:]


def _mutate(text, edits):
    for old, new, count in edits:
        assert text.count(old) == count, "mutation site not found as expected: %r" % old
        text = text.replace(old, new)
    return text


def test_every_planted_mistake_fails_a_pin(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    text = _source()
    jobs = [("unmodified", _build(text, str(tmp_path), "unmodified"), False)]
    for i, (what, edits) in enumerate(MUTANTS):
        jobs.append((what, _build(_mutate(text, edits), str(tmp_path), "mutant%02d" % i), True))
    with ThreadPoolExecutor(max_workers=6) as pool:
        results = list(pool.map(lambda j: (j[0], j[2]) + _run_pins(j[1], j[2]), jobs))
    control = results[0]
    assert control[2] == 0, "the unmodified oracle build fails its pins:\n" + control[3]
    survivors = [what for what, is_mutant, rc, _ in results[1:] if rc == 0]
    crashed = [(what, rc) for what, is_mutant, rc, _ in results[1:] if rc not in (0, 1)]
    assert not survivors, "planted mistakes that no pin catches: %s" % survivors
    assert not crashed, "mutants that did not fail by assertion: %s" % crashed
