/*
 * kvq_oracle.c -- plain, slow, scalar CPU oracle for the KV-cache format
 * conversions.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product library never does, and
 * this file shares no code, header, table or helper with the HIP library.
 *
 * What is computed follows the page "Implementation: Turboderp org Exllamav2
 * Ext Cache" (sections Description, Signature and I/O Contract), which names
 * the five operations, their arguments (batch_size, offset, width, page_size,
 * cache_seqlens, block_table, wbits) and the two cache layouts, but leaves the
 * numerics open.  The numeric conventions taken here are:
 *   - blocks of 32 consecutive elements along head_dim, one fp16 scale each;
 *   - symmetric absmax scale  s = absmax / (2^(b-1) - 1)  divided in fp32,
 *     stored as fp16 with round-half-to-even (subnormals kept);
 *   - code  q = clamp(round_half_even(x / s16), -2^(b-1), 2^(b-1) - 1)  with
 *     the fp32 quotient and the *stored* fp16 scale, q = 0 when s16 == 0;
 *     stored offset-binary  u = q + 2^(b-1);
 *   - packing as one little-endian bit stream per token row: code j of the
 *     row occupies bits [b*j, b*j + b) (4-bit: 8 codes per uint32 word,
 *     6-bit: 16 codes per 12 bytes, 8-bit: one code per byte);
 *   - dequantization x' = fp16_rne((float)q * (float)s16);
 *   - the page's unsigned 8-bit FP8 format = the high byte of the fp16 bit pattern (e5m2 by
 *     truncation toward zero); back: byte << 8;
 *   - count_match: number of leading equal elements of the two arrays within
 *     min(max_a, len_a, len_b), one element at a time;
 *   - extensions: b = 8 block codes (the page's Usage section lists a Q8
 *     cache), a format per tensor (fp8 high byte or Q4/Q6/Q8 for K and for
 *     V, contiguous or paged), the widen of every cached position
 *     [0, cache_seqlens[b] + width) of each sequence, and bytes per token.
 * Every step is written out plainly, one element at a time; no blocking,
 * vectorisation or reordering beyond the definition.
 *
 * Below, "[Cache]" stands for that page; each function names the section
 * (and, where the page is silent, the reading above) it follows.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared (IEEE-754
 * binary32 arithmetic through SSE, round-to-nearest-even, no FTZ/DAZ).
 *
 * Parity pins: every function here is pinned by the CPU test-suite against
 * values fixed independently of this file (exhaustive comparison with
 * numpy's float16 conversion, exact rational arithmetic, brute-force argmin,
 * hand-derived bit patterns, closed forms).  See the test modules named
 * test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16, from the format definition.                            */
/* ------------------------------------------------------------------------ */

/* Exact value of an fp16 bit pattern (every fp16 value is exact in double).
 * IEEE-754 binary16 definition; [Cache] I/O Contract names the fp16 (kHalf)
 * caches this decodes. */
double orc_f16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    } else {
        v = ldexp((double)(1024 + m), e - 25);     /* (1.m) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a non-negative double that is an exact multiple of some power of two
 * (any double is) to the nearest integer, ties to even. */
static double round_half_even_nonneg(double n)
{
    double fl = floor(n);
    double frac = n - fl;            /* exact: n and fl share the exponent range */
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Correctly rounded (round-half-to-even) conversion of a double to fp16,
 * with gradual underflow and overflow to infinity.  IEEE-754 binary16
 * rounding; the reading of [Cache] stores scales and dequantized values as
 * fp16 under this rounding. */
uint16_t orc_f16_encode_rne(double v)
{
    if (isnan(v)) return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    /* Largest finite fp16 is 65504 = (2 - 2^-10) * 2^15; the rounding
     * boundary to the next (unrepresentable) value 65536 is 65520, and a
     * tie there rounds to the even neighbour, which is 65536 -> infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);
    int E;
    frexp(a, &E);                    /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                   /* a in [2^e, 2^(e+1)) */
    if (e < -14) {
        /* subnormal range: quantum 2^-24 */
        double k = round_half_even_nonneg(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)k);   /* k == 1024 is the min normal */
    }
    /* normal range: 11 significant bits, quantum 2^(e-10) */
    double k = round_half_even_nonneg(ldexp(a, 10 - e));   /* in [1024, 2048] */
    uint32_t bits = ((uint32_t)(e + 15) << 10) + ((uint32_t)k - 1024u);
    /* k == 2048 carries into the exponent field, which is the right value */
    return (uint16_t)(sign | bits);
}

/* ------------------------------------------------------------------------ */
/* 8-bit format: the high byte of the fp16 pattern.                          */
/* ------------------------------------------------------------------------ */

/* [Cache] Description of fp16_to_fp8 / fp8_to_fp16 and I/O Contract (the
 * unsigned 8-bit cache), read as the high byte of the fp16 pattern. */
uint8_t orc_fp8_from_f16(uint16_t h) { return (uint8_t)(h >> 8); }
uint16_t orc_f16_from_fp8(uint8_t b) { return (uint16_t)((uint16_t)b << 8); }

/* ------------------------------------------------------------------------ */
/* Block quantization.                                                       */
/* ------------------------------------------------------------------------ */

static int qmax_of(int wbits) { return (1 << (wbits - 1)) - 1; }   /* Q */
static int zero_of(int wbits) { return 1 << (wbits - 1); }         /* Z */

/* [Cache] Description of fp16_to_q_kv and I/O Contract (per-block scale
 * factors), with the scale reading above.
 * Scale of a block from its absmax a (an fp16 pattern, a >= 0):
 * s32 = a / Q in fp32, stored as fp16 round-half-even. */
uint16_t orc_scale_from_absmax(uint16_t a_bits, int wbits)
{
    float a = (float)orc_f16_decode(a_bits);
    float s32 = a / (float)qmax_of(wbits);
    return orc_f16_encode_rne((double)s32);
}

/* Offset-binary codes of n elements under a given stored scale.  [Cache]
 * Description of fp16_to_q_kv (wbits-bit codes), with the code reading
 * above. */
void orc_quant_elems(const uint16_t* x, int64_t n, uint16_t s16, int wbits, uint8_t* u)
{
    const int Z = zero_of(wbits);
    const float sf = (float)orc_f16_decode(s16);
    for (int64_t i = 0; i < n; ++i) {
        int q;
        if (sf == 0.0f) {
            q = 0;
        } else {
            float xf = (float)orc_f16_decode(x[i]);
            float v = xf / sf;                   /* fp32 quotient */
            float r = nearbyintf(v);             /* ties to even (default mode) */
            if (r < (float)(-Z)) r = (float)(-Z);
            if (r > (float)(Z - 1)) r = (float)(Z - 1);
            q = (int)r;
        }
        u[i] = (uint8_t)(q + Z);
    }
}

/* One block of L elements: absmax -> scale -> codes ([Cache] Description of
 * fp16_to_q_kv: block quantization). */
void orc_quant_block(const uint16_t* x, int L, int wbits, uint16_t* s16_out, uint8_t* u_out)
{
    /* absmax; -0 counts as 0.  The maximum of |x| is taken on the values. */
    double amax = 0.0;
    uint16_t a_bits = 0;
    for (int i = 0; i < L; ++i) {
        double m = fabs(orc_f16_decode(x[i]));
        if (m > amax) {
            amax = m;
            a_bits = (uint16_t)(x[i] & 0x7FFF);
        }
    }
    uint16_t s16 = orc_scale_from_absmax(a_bits, wbits);
    *s16_out = s16;
    orc_quant_elems(x, L, s16, wbits, u_out);
}

/* Dequantize n offset-binary codes with one stored scale ([Cache]
 * Description of q_to_fp16_kv, with the dequantization reading above). */
void orc_dequant_elems(const uint8_t* u, int64_t n, uint16_t s16, int wbits, uint16_t* out)
{
    const int Z = zero_of(wbits);
    const float sf = (float)orc_f16_decode(s16);
    for (int64_t i = 0; i < n; ++i) {
        int q = (int)u[i] - Z;
        float prod = (float)q * sf;              /* exact: |q| <= 32, 11-bit sf */
        out[i] = orc_f16_encode_rne((double)prod);
    }
}

/* ------------------------------------------------------------------------ */
/* Packing: one little-endian bit stream; code j at bits [b*j, b*j + b).      */
/* ([Cache] I/O Contract: packed wbits-bit codes; the bit order is the       */
/* reading above.)                                                           */
/* ------------------------------------------------------------------------ */

void orc_pack_bits(const uint8_t* u, int64_t n, int wbits, uint8_t* out)
{
    int64_t nbytes = (n * wbits + 7) / 8;
    memset(out, 0, (size_t)nbytes);
    for (int64_t j = 0; j < n; ++j) {
        for (int k = 0; k < wbits; ++k) {
            int64_t bit = j * wbits + k;
            if ((u[j] >> k) & 1)
                out[bit / 8] |= (uint8_t)(1u << (bit % 8));
        }
    }
}

void orc_unpack_bits(const uint8_t* in, int64_t n, int wbits, uint8_t* u)
{
    for (int64_t j = 0; j < n; ++j) {
        int v = 0;
        for (int k = 0; k < wbits; ++k) {
            int64_t bit = j * wbits + k;
            if ((in[bit / 8] >> (bit % 8)) & 1)
                v |= 1 << k;
        }
        u[j] = (uint8_t)v;
    }
}

/* ------------------------------------------------------------------------ */
/* Token rows of R = heads * head_dim elements (R a multiple of 32).         */
/* codes row: R * wbits / 8 bytes; scales row: R / 32 fp16.                  */
/* ------------------------------------------------------------------------ */

#define ORC_BLOCK 32

void orc_quant_rows(const uint16_t* in, int64_t n_rows, int R, int wbits,
                    uint8_t* codes, uint16_t* scales)
{
    uint8_t u[4096];
    const int64_t code_bytes = (int64_t)R * wbits / 8;
    for (int64_t r = 0; r < n_rows; ++r) {
        const uint16_t* x = in + r * R;
        uint8_t* crow = codes + r * code_bytes;
        uint16_t* srow = scales + r * (R / ORC_BLOCK);
        /* the row's code stream is built in pieces of at most 4096 codes */
        for (int base = 0; base < R; base += 4096) {
            int len = (R - base < 4096) ? (R - base) : 4096;
            for (int blk = 0; blk < len / ORC_BLOCK; ++blk) {
                int j0 = base + blk * ORC_BLOCK;
                orc_quant_block(x + j0, ORC_BLOCK, wbits, &srow[j0 / ORC_BLOCK],
                                u + blk * ORC_BLOCK);
            }
            orc_pack_bits(u, len, wbits, crow + (int64_t)base * wbits / 8);
        }
    }
}

void orc_dequant_rows(const uint8_t* codes, const uint16_t* scales, int64_t n_rows,
                      int R, int wbits, uint16_t* out)
{
    uint8_t u[4096];
    const int64_t code_bytes = (int64_t)R * wbits / 8;
    for (int64_t r = 0; r < n_rows; ++r) {
        const uint8_t* crow = codes + r * code_bytes;
        const uint16_t* srow = scales + r * (R / ORC_BLOCK);
        uint16_t* y = out + r * R;
        for (int base = 0; base < R; base += 4096) {
            int len = (R - base < 4096) ? (R - base) : 4096;
            orc_unpack_bits(crow + (int64_t)base * wbits / 8, len, wbits, u);
            for (int blk = 0; blk < len / ORC_BLOCK; ++blk) {
                int j0 = base + blk * ORC_BLOCK;
                orc_dequant_elems(u + blk * ORC_BLOCK, ORC_BLOCK, srow[j0 / ORC_BLOCK],
                                  wbits, y + j0);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Which cache row (b, t) of the call maps to.                               */
/* Contiguous (page_size == 0): row (b, offset + t) of a [dim0, dim1] grid.   */
/* Paged: position p = cache_seqlens[b] + offset + t of sequence b lives in   */
/* physical page block_table[b][p / page_size], slot p % page_size.           */
/* Returns the flat row index dim1 * d0 + d1, or -1 when the row is skipped   */
/* (p < 0, page index past the table, or page outside [0, dim0)).             */
/* ------------------------------------------------------------------------ */

/* [Cache] Description (contiguous windows and the paged layout addressed
 * through block_table / cache_seqlens) and Signature (batch_size, offset,
 * width, page_size). */
int64_t orc_resolve_row(int b, int t, int dim0, int dim1, int offset, int page_size,
                        const int32_t* cache_seqlens, const int32_t* block_table,
                        int bt_cols)
{
    if (page_size == 0)
        return (int64_t)b * dim1 + offset + t;
    int64_t p = (int64_t)cache_seqlens[b] + offset + t;
    if (p < 0) return -1;
    int64_t pi = p / page_size;
    if (pi >= bt_cols) return -1;
    int64_t page = block_table[(int64_t)b * bt_cols + pi];
    if (page < 0 || page >= dim0) return -1;
    return page * page_size + p % page_size;
}

/* Rows touched by one call, in (b, t) order; returns their count
 * (rows[i] = -1 marks a skipped row). */
int64_t orc_call_rows(int dim0, int dim1, int batch_size, int offset, int width,
                      int page_size, const int32_t* cache_seqlens,
                      const int32_t* block_table, int bt_cols, int64_t* rows)
{
    int64_t n = 0;
    for (int b = 0; b < batch_size; ++b)
        for (int t = 0; t < width; ++t)
            rows[n++] = orc_resolve_row(b, t, dim0, dim1, offset, page_size,
                                        cache_seqlens, block_table, bt_cols);
    return n;
}

/* ------------------------------------------------------------------------ */
/* Cache-level operations, same argument meaning as the library calls.       */
/* Host buffers; a NULL K or V triple skips that half.                        */
/* ------------------------------------------------------------------------ */

/* [Cache] Description / Signature of fp16_to_q_kv: K and V together. */
void orc_fp16_to_q_kv(const uint16_t* k_in, uint8_t* k_out, uint16_t* k_scales,
                      const uint16_t* v_in, uint8_t* v_out, uint16_t* v_scales,
                      int dim0, int dim1, int heads, int head_dim,
                      int batch_size, int offset, int width, int page_size,
                      const int32_t* cache_seqlens, const int32_t* block_table,
                      int bt_cols, int wbits)
{
    const int R = heads * head_dim;
    const int64_t cb = (int64_t)R * wbits / 8, sb = R / ORC_BLOCK;
    for (int b = 0; b < batch_size; ++b) {
        for (int t = 0; t < width; ++t) {
            int64_t row = orc_resolve_row(b, t, dim0, dim1, offset, page_size,
                                          cache_seqlens, block_table, bt_cols);
            if (row < 0) continue;
            if (k_in)
                orc_quant_rows(k_in + row * R, 1, R, wbits, k_out + row * cb, k_scales + row * sb);
            if (v_in)
                orc_quant_rows(v_in + row * R, 1, R, wbits, v_out + row * cb, v_scales + row * sb);
        }
    }
}

/* [Cache] Description / Signature of q_to_fp16_kv: the inverse over the
 * same rows. */
void orc_q_to_fp16_kv(const uint8_t* k_in, uint16_t* k_out, const uint16_t* k_scales,
                      const uint8_t* v_in, uint16_t* v_out, const uint16_t* v_scales,
                      int dim0, int dim1, int heads, int head_dim,
                      int batch_size, int offset, int width, int page_size,
                      const int32_t* cache_seqlens, const int32_t* block_table,
                      int bt_cols, int wbits)
{
    const int R = heads * head_dim;
    const int64_t cb = (int64_t)R * wbits / 8, sb = R / ORC_BLOCK;
    for (int b = 0; b < batch_size; ++b) {
        for (int t = 0; t < width; ++t) {
            int64_t row = orc_resolve_row(b, t, dim0, dim1, offset, page_size,
                                          cache_seqlens, block_table, bt_cols);
            if (row < 0) continue;
            if (k_in)
                orc_dequant_rows(k_in + row * cb, k_scales + row * sb, 1, R, wbits, k_out + row * R);
            if (v_in)
                orc_dequant_rows(v_in + row * cb, v_scales + row * sb, 1, R, wbits, v_out + row * R);
        }
    }
}

/* fp16 <-> 8-bit over the contiguous window rows (b, offset .. offset+width):
 * [Cache] Description / Signature of fp16_to_fp8 and fp8_to_fp16. */
void orc_fp16_to_fp8_cache(const uint16_t* in, uint8_t* out, int dim0, int dim1,
                           int heads, int head_dim, int batch_size, int offset, int width)
{
    (void)dim0;
    const int64_t R = (int64_t)heads * head_dim;
    for (int b = 0; b < batch_size; ++b)
        for (int t = 0; t < width; ++t) {
            int64_t row = (int64_t)b * dim1 + offset + t;
            for (int64_t j = 0; j < R; ++j)
                out[row * R + j] = orc_fp8_from_f16(in[row * R + j]);
        }
}

void orc_fp8_to_fp16_cache(const uint8_t* in, uint16_t* out, int dim0, int dim1,
                           int heads, int head_dim, int batch_size, int offset, int width)
{
    (void)dim0;
    const int64_t R = (int64_t)heads * head_dim;
    for (int b = 0; b < batch_size; ++b)
        for (int t = 0; t < width; ++t) {
            int64_t row = (int64_t)b * dim1 + offset + t;
            for (int64_t j = 0; j < R; ++j)
                out[row * R + j] = orc_f16_from_fp8(in[row * R + j]);
        }
}

/* ------------------------------------------------------------------------ */
/* Matching prefix length, one element at a time (elements of 4 or 8 bytes). */
/* [Cache] Description of count_match, with the element reading above.      */
/* ------------------------------------------------------------------------ */

int64_t orc_count_match(const void* a, int64_t len_a, const void* b, int64_t len_b,
                        int64_t max_a, int elem_bytes)
{
    int64_t n = max_a;
    if (n > len_a) n = len_a;
    if (n > len_b) n = len_b;
    if (n < 0) n = 0;
    const unsigned char* pa = (const unsigned char*)a;
    const unsigned char* pb = (const unsigned char*)b;
    for (int64_t i = 0; i < n; ++i)
        if (memcmp(pa + i * elem_bytes, pb + i * elem_bytes, (size_t)elem_bytes) != 0)
            return i;
    return n;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the fp16 codec and the scale rule (loops over the scalar   */
/* functions above; for exhaustive tests).                                   */
/* ------------------------------------------------------------------------ */

void orc_f16_decode_array(const uint16_t* h, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_decode(h[i]);
}

void orc_f16_encode_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_encode_rne(v[i]);
}

void orc_scale_array(const uint16_t* a_bits, int64_t n, int wbits, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_scale_from_absmax(a_bits[i], wbits);
}

/* ------------------------------------------------------------------------ */
/* Per-tensor formats (K and V may differ) and the full-prefix dequantize.   */
/* fmt 0 = 8-bit high byte (no scales); 4, 6, 8 = block codes + fp16 scales. */
/* Extensions of [Cache]'s operations (its Usage section names 8-bit caching */
/* and Q4, Q6 and Q8 cache classes): the per-row rules above, with a format  */
/* chosen per tensor.                                                        */
/* ------------------------------------------------------------------------ */

static void orc_narrow_row(const uint16_t* x, int64_t R, int fmt, uint8_t* out, uint16_t* scales)
{
    if (fmt == 0) {
        for (int64_t j = 0; j < R; ++j) out[j] = orc_fp8_from_f16(x[j]);
    } else {
        orc_quant_rows(x, 1, (int)R, fmt, out, scales);
    }
}

static void orc_widen_row(const uint8_t* in, const uint16_t* scales, int64_t R, int fmt, uint16_t* out)
{
    if (fmt == 0) {
        for (int64_t j = 0; j < R; ++j) out[j] = orc_f16_from_fp8(in[j]);
    } else {
        orc_dequant_rows(in, scales, 1, (int)R, fmt, out);
    }
}

/* bytes of one row's compact form, and of its scales */
static int64_t orc_fmt_row_bytes(int64_t R, int fmt) { return fmt == 0 ? R : R * fmt / 8; }
static int64_t orc_fmt_scale_count(int64_t R, int fmt) { return fmt == 0 ? 0 : R / ORC_BLOCK; }

void orc_fp16_to_kv(const uint16_t* k_in, uint8_t* k_out, uint16_t* k_scales, int fmt_k,
                    const uint16_t* v_in, uint8_t* v_out, uint16_t* v_scales, int fmt_v,
                    int dim0, int dim1, int heads, int head_dim,
                    int batch_size, int offset, int width, int page_size,
                    const int32_t* cache_seqlens, const int32_t* block_table, int bt_cols)
{
    const int64_t R = (int64_t)heads * head_dim;
    for (int b = 0; b < batch_size; ++b)
        for (int t = 0; t < width; ++t) {
            int64_t row = orc_resolve_row(b, t, dim0, dim1, offset, page_size,
                                          cache_seqlens, block_table, bt_cols);
            if (row < 0) continue;
            if (k_in)
                orc_narrow_row(k_in + row * R, R, fmt_k, k_out + row * orc_fmt_row_bytes(R, fmt_k),
                               k_scales ? k_scales + row * orc_fmt_scale_count(R, fmt_k) : 0);
            if (v_in)
                orc_narrow_row(v_in + row * R, R, fmt_v, v_out + row * orc_fmt_row_bytes(R, fmt_v),
                               v_scales ? v_scales + row * orc_fmt_scale_count(R, fmt_v) : 0);
        }
}

static void orc_widen_kv_row(int64_t row, int64_t R,
                             const uint8_t* k_in, uint16_t* k_out, const uint16_t* k_scales, int fmt_k,
                             const uint8_t* v_in, uint16_t* v_out, const uint16_t* v_scales, int fmt_v)
{
    if (k_in)
        orc_widen_row(k_in + row * orc_fmt_row_bytes(R, fmt_k),
                      k_scales ? k_scales + row * orc_fmt_scale_count(R, fmt_k) : 0, R, fmt_k,
                      k_out + row * R);
    if (v_in)
        orc_widen_row(v_in + row * orc_fmt_row_bytes(R, fmt_v),
                      v_scales ? v_scales + row * orc_fmt_scale_count(R, fmt_v) : 0, R, fmt_v,
                      v_out + row * R);
}

void orc_kv_to_fp16(const uint8_t* k_in, uint16_t* k_out, const uint16_t* k_scales, int fmt_k,
                    const uint8_t* v_in, uint16_t* v_out, const uint16_t* v_scales, int fmt_v,
                    int dim0, int dim1, int heads, int head_dim,
                    int batch_size, int offset, int width, int page_size,
                    const int32_t* cache_seqlens, const int32_t* block_table, int bt_cols)
{
    const int64_t R = (int64_t)heads * head_dim;
    for (int b = 0; b < batch_size; ++b)
        for (int t = 0; t < width; ++t) {
            int64_t row = orc_resolve_row(b, t, dim0, dim1, offset, page_size,
                                          cache_seqlens, block_table, bt_cols);
            if (row < 0) continue;
            orc_widen_kv_row(row, R, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v);
        }
}

/* Paged row of position p of sequence b (p counted from the start of the
 * sequence), or -1 (past the table, or page outside [0, dim0)). */
static int64_t orc_paged_position(int b, int64_t p, int dim0, int page_size,
                                  const int32_t* block_table, int bt_cols)
{
    int64_t pi = p / page_size;
    if (pi >= bt_cols) return -1;
    int64_t page = block_table[(int64_t)b * bt_cols + pi];
    if (page < 0 || page >= dim0) return -1;
    return page * page_size + p % page_size;
}

/* Rows of the full prefix of each sequence: positions
 * p in [0, min(cache_seqlens[b] + width, max_len)), in (b, p) order, with
 * -1 for skipped positions; returns their count. */
int64_t orc_prefix_rows(int dim0, int page_size, int batch_size, int width, int max_len,
                        const int32_t* cache_seqlens, const int32_t* block_table, int bt_cols,
                        int64_t* rows)
{
    int64_t n = 0;
    for (int b = 0; b < batch_size; ++b) {
        int64_t end = (int64_t)cache_seqlens[b] + width;
        if (end > max_len) end = max_len;
        for (int64_t p = 0; p < end; ++p)
            rows[n++] = orc_paged_position(b, p, dim0, page_size, block_table, bt_cols);
    }
    return n;
}

void orc_kv_to_fp16_prefix(const uint8_t* k_in, uint16_t* k_out, const uint16_t* k_scales, int fmt_k,
                           const uint8_t* v_in, uint16_t* v_out, const uint16_t* v_scales, int fmt_v,
                           int dim0, int dim1, int heads, int head_dim,
                           int batch_size, int width, int max_len,
                           const int32_t* cache_seqlens, const int32_t* block_table, int bt_cols)
{
    const int64_t R = (int64_t)heads * head_dim;
    for (int b = 0; b < batch_size; ++b) {
        int64_t end = (int64_t)cache_seqlens[b] + width;
        if (end > max_len) end = max_len;
        for (int64_t p = 0; p < end; ++p) {
            int64_t row = orc_paged_position(b, p, dim0, dim1, block_table, bt_cols);
            if (row < 0) continue;
            orc_widen_kv_row(row, R, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v);
        }
    }
}

/* Bytes one token occupies in one cache tensor of a format (the capacity
 * arithmetic of the llama.cpp tensor-split planning page, applied to these
 * formats):
 * 16 = fp16, 0 = 8-bit high byte, 4/6/8 = block codes + one fp16 per 32. */
int64_t orc_bytes_per_token(int fmt, int heads, int head_dim)
{
    const int64_t R = (int64_t)heads * head_dim;
    if (fmt == 16) return 2 * R;
    return orc_fmt_row_bytes(R, fmt) + 2 * orc_fmt_scale_count(R, fmt);
}
