// kvq_device.h -- gfx950 device building blocks of the KV-cache conversions.
//
// A "chunk" is 8 consecutive fp16 elements of a token row (one 128-bit
// load).  When quantizing, a lane holds two consecutive chunks and a lane
// pair one 32-element block, so the block absmax is one DPP exchange inside
// the wave (no LDS).
//
// Arithmetic definitions (ExLlamaV2 cache page, Description of fp16_to_q_kv /
// q_to_fp16_kv; the numeric reading is stated in kvq.h):
//   scale  s16 = fp16_rne(absmax / Q),  Q = 2^(b-1) - 1
//   code   q = clamp(round_half_even(x / s16), -Z, Z-1), Z = 2^(b-1); u = q + Z
//   value  x' = fp16_rne(q * s16)
// How each is computed here without a per-element IEEE divide is described
// next to the function that does it.
//
// (The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
// Exllamav2 Ext Cache".)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
    return (float)h;
}

// fp32 -> fp16 bits, round to nearest even, subnormals kept (v_cvt_f16_f32
// under the default MODE: round-nearest-even, fp16 denormals enabled).
__device__ __forceinline__ uint32_t f2h(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ half2_t as_h2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// ---------------------------------------------------------------- reductions

// DPP quad_perm control [1,0,3,2]: each lane reads its pair partner (lane ^ 1).
constexpr int kPairSwap = 0xB1;

// Max over a lane pair (lanes 2m, 2m+1), both active together.
__device__ __forceinline__ uint32_t pair_max(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kPairSwap, 0xF, 0xF, false);
    return v > o ? v : o;
}

// Running magnitude maximum per fp16 half: max(acc, w, -w) = max(acc, |w|)
// in one v_pk_maximum3_f16 (third source negated in both halves).  This is
// the IEEE 754-2019 maximum, so a zero of either sign gives +0; for finite
// fp16 (the quantizer's domain; fp16 denormals are kept) the result is the
// largest magnitude, and such non-negative values order like their bits.
__device__ __forceinline__ uint32_t absmax_step(uint32_t acc, uint32_t w) {
    uint32_t d;
    asm("v_pk_maximum3_f16 %0, %1, %2, %2 neg_lo:[0,0,1] neg_hi:[0,0,1]" : "=v"(d) : "v"(acc), "v"(w));
    return d;
}

// Largest |x| of the 2N fp16 values in words w[0..N), N even, as fp16 bits:
// two interleaved chains of absmax_step, then an integer max of the
// non-negative halves.
template <int N>
__device__ __forceinline__ uint32_t absmax_words(const uint32_t (&w)[N]) {
    static_assert(N >= 2 && N % 2 == 0, "an even number of words");
    uint32_t a = absmax_step(w[0], w[0]);
    uint32_t b = absmax_step(w[1], w[1]);
#pragma unroll
    for (int i = 2; i < N; i += 2) {
        a = absmax_step(a, w[i]);
        b = absmax_step(b, w[i + 1]);
    }
    const u16x2_t m = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b));
    return (uint32_t)(m.x > m.y ? m.x : m.y);
}

// Largest |x| of the 16 fp16 values of two chunks, as fp16 bits.
__device__ __forceinline__ uint32_t absmax_2chunks(uint4 v, uint4 w) {
    const uint32_t x[8] = {v.x, v.y, v.z, v.w, w.x, w.y, w.z, w.w};
    return absmax_words(x);
}

// ---------------------------------------------------------------- scale

// s16 = fp16_rne(a / Q) computed as fp16_rne(a * fl32(1/Q)).  For every
// finite fp16 a and Q in {7, 31, 127} (4-, 6- and 8-bit codes) this equals
// the correctly rounded a/Q: the product is within 1.5 ulp32 of a/Q, and a/Q
// is never that close to an fp16 rounding boundary unless it is exactly
// representable.  The GPU test of the scale rule checks all 31,744 finite
// fp16 absmax values at each of the three widths against the oracle's
// divide.
template <int WBITS>
__device__ __forceinline__ uint32_t scale_from_absmax(uint32_t a_bits) {
    constexpr float kInvQ = 1.0f / (float)((1 << (WBITS - 1)) - 1);
    return f2h(h2f(a_bits) * kInvQ);
}

// ---------------------------------------------------------------- quantize

// y = x * r with x one fp16 half of a word (low or high), r fp32, in one
// v_fma_mix_f32 (the f16 operand is widened exactly inside the instruction;
// the +0 addend only affects the sign of a zero product, which no code
// depends on).
__device__ __forceinline__ float mul_f16lo(uint32_t w, float r) {
    float y;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(y) : "v"(w), "v"(r));
    return y;
}
__device__ __forceinline__ float mul_f16hi(uint32_t w, float r) {
    float y;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(y) : "v"(w), "v"(r));
    return y;
}

// Operands derived once per block from its stored scale s16.
struct ScaleOps {
    float s;        // scale (1 for a zero scale)
    float r;        // rcp(s), within 1 ulp of 1/s (0 for a zero scale)
    uint32_t r2;    // fp16(r) in both halves; used only for normal scales
};

// A zero scale maps every element to q = 0: with (s, r) = (1, 0) the
// quotient below is 0 for every finite x.
__device__ __forceinline__ ScaleOps prep_scale(uint32_t s16) {
    const float sf = h2f(s16);
    const bool zero = (sf == 0.0f);
    ScaleOps o;
    o.s = zero ? 1.0f : sf;
    o.r = zero ? 0.0f : __builtin_amdgcn_rcpf(sf);
    const uint32_t r16 = f2h(o.r);
    o.r2 = r16 | (r16 << 16);
    return o;
}

// Code of one element; the low WBITS bits of the result are u = q + Z, the
// bits from 24 up hold the exponent of the rounding constant (bits WBITS..23
// are zero).
//
// q = round_half_even(x / s) is obtained without a divide, from a first
// quotient y refined by one exact residual:
//   e  = fma(-y, s, x)        exact: y*s is within a few ulp of x
//   y2 = fma(e, r, y)         r = rcp(s), within 1 ulp of 1/s
// For fp16 x and s, x/s is either an exact half-integer tie (then y2 lands
// on it exactly: the correction's own error is far below half an ulp) or
// lies at least ~2^-13 relative from any tie, far beyond the few-ulp error
// of y2; so rounding y2 gives round_half_even(x / s) on every pair.
// Adding M = 2^23 + Z rounds to an integer with ties-to-even (the fp32 ulp
// in [2^23, 2^24) is 1; Z is even, so parity is kept) and leaves u in the
// low mantissa bits.
//
// Two paths, chosen per block:
//  - normal scale (s16 >= 2^-14): the first quotient is one packed fp16
//    multiply y = fp16(x * fp16(r)) for two elements (relative error below
//    2^-9; the residual x - y*s then still fits 24 bits, so e is exact), and
//    no clamp: a normal s16 = fp16_rne(a / Q) is at least (a / Q)(1 - 2^-11),
//    so every element of its block has |x / s16| <= Q (1 + 2^-10) < Q + 1/2,
//    which keeps y2 + M in [2^23, 2^24) and the code in [-Q, Q];
//  - subnormal or zero scale: y = x * r in fp32 and the clamp to [-Z, Z-1]
//    (which commutes with rounding: integer bounds).
// The normal path is only valid on that domain (|x / s| < Q + 1/2).

// e = fma(-y, s, x) and y2 = fma(e, r, y) with y an fp16 half of yw and x an
// fp16 half of xw (HI selects the high halves), in two v_fma_mix_f32.
template <bool HI>
__device__ __forceinline__ float refine_h(uint32_t yw, uint32_t xw, float s, float r) {
    float e, y2;
    if (HI) {
        asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(e) : "v"(yw), "v"(s), "v"(xw));
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "=v"(y2) : "v"(e), "v"(r), "v"(yw));
    } else {
        asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel_hi:[1,0,1]" : "=v"(e) : "v"(yw), "v"(s), "v"(xw));
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,0,1]" : "=v"(y2) : "v"(e), "v"(r), "v"(yw));
    }
    return y2;
}

// Same refinement with an fp32 first quotient y (x an fp16 half of xw).
template <bool HI>
__device__ __forceinline__ float refine_f(float y, uint32_t xw, float s, float r) {
    float e;
    if (HI)
        asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "=v"(e) : "v"(y), "v"(s), "v"(xw));
    else
        asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel_hi:[0,0,1]" : "=v"(e) : "v"(y), "v"(s), "v"(xw));
    return __builtin_fmaf(e, r, y);
}

template <int WBITS>
__device__ __forceinline__ uint32_t round_code(float y2) {
    constexpr float Z = (float)(1 << (WBITS - 1));
    return __builtin_bit_cast(uint32_t, y2 + (8388608.0f + Z));
}

template <int WBITS>
__device__ __forceinline__ uint32_t round_code_clamped(float y2) {
    constexpr float Z = (float)(1 << (WBITS - 1));
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(y2, -Z, Z - 1.0f) + (8388608.0f + Z));
}

// Normal-scale path for the 8 elements of a chunk.
template <int WBITS>
__device__ __forceinline__ void quant_chunk_normal(uint4 v, const ScaleOps& so, uint32_t (&u)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t yw = as_u32(as_h2(w[i]) * as_h2(so.r2));
        u[2 * i] = round_code<WBITS>(refine_h<false>(yw, w[i], so.s, so.r));
        u[2 * i + 1] = round_code<WBITS>(refine_h<true>(yw, w[i], so.s, so.r));
    }
}

// Clamping path (subnormal or zero scale; defined on every finite pair).
template <int WBITS>
__device__ __forceinline__ void quant_chunk_clamped(uint4 v, const ScaleOps& so, uint32_t (&u)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u[2 * i] = round_code_clamped<WBITS>(refine_f<false>(mul_f16lo(w[i], so.r), w[i], so.s, so.r));
        u[2 * i + 1] = round_code_clamped<WBITS>(refine_f<true>(mul_f16hi(w[i], so.r), w[i], so.s, so.r));
    }
}

// The kernels' dispatch: s16 is the block's stored scale (fp16 bits).
template <int WBITS>
__device__ __forceinline__ void quant_chunk(uint4 v, uint32_t s16, const ScaleOps& so, uint32_t (&u)[8]) {
    if (s16 >= 0x0400u) quant_chunk_normal<WBITS>(v, so, u);
    else quant_chunk_clamped<WBITS>(v, so, u);
}

// The same for N chunks of one block, with one branch for the block.
template <int WBITS, int N>
__device__ __forceinline__ void quant_chunks(const uint4 (&v)[N], uint32_t s16, const ScaleOps& so,
                                             uint32_t (&u)[N][8]) {
    if (s16 >= 0x0400u) {
#pragma unroll
        for (int k = 0; k < N; ++k) quant_chunk_normal<WBITS>(v[k], so, u[k]);
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) quant_chunk_clamped<WBITS>(v[k], so, u[k]);
    }
}

// 4-bit: code j at bits 4j..4j+3 of one little-endian word.  Each u[j] is
// 0x4B000000 + code (the rounding constant's exponent above zero bits
// 4..23), and the fields do not overlap, so the word is the sum of the u[j]
// shifted into place (shift-adds, mod 2^32) less the exponent terms that
// stay inside 32 bits: 0x4B000000 from u[0] and 0xB0000000 from u[1] << 4
// (those of the higher codes shift out), i.e. plus 0x05000000.
// (a << SH) + b in one v_lshl_add_u32 (the compiler would otherwise split
// such chains into shifts and three-input adds).
template <int SH>
__device__ __forceinline__ uint32_t lshl_add(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "n"(SH), "v"(b));
    return d;
}

__device__ __forceinline__ uint32_t pack_q4(const uint32_t (&u)[8]) {
    const uint32_t t01 = lshl_add<4>(u[1], u[0]);
    const uint32_t t23 = lshl_add<4>(u[3], u[2]);
    const uint32_t t45 = lshl_add<4>(u[5], u[4]);
    const uint32_t t67 = lshl_add<4>(u[7], u[6]);
    const uint32_t lo = lshl_add<8>(t23, t01);      // exponent terms of u[2], u[3] shift out
    const uint32_t hi = lshl_add<8>(t67, t45);
    return lshl_add<16>(hi, lo) + 0x05000000u;      // those of hi shift out
}

// 6-bit: code j at bits 6j..6j+5 of a 48-bit little-endian field, returned
// as (lo32, hi) where only the low 16 bits of hi are meaningful.
__device__ __forceinline__ void pack_q6(const uint32_t (&u)[8], uint32_t& lo, uint32_t& hi) {
    uint32_t w = (u[2] << 12) | (u[3] << 18) | (u[4] << 24) | (u[5] << 30);
    const uint32_t t = u[0] | (u[1] << 6);
    lo = (t & 0xFFFu) | w;
    hi = (u[5] >> 2) | (u[6] << 4) | (u[7] << 10);
}

// 8-bit block codes: code j is byte j; four codes per word, assembled with
// byte permutes from the low bytes of the element results.
__device__ __forceinline__ uint32_t pack_q8x4(uint32_t u0, uint32_t u1, uint32_t u2, uint32_t u3) {
    const uint32_t t01 = __builtin_amdgcn_perm(u1, u0, 0x00000400u);   // [u0.b0, u1.b0, -, -]
    const uint32_t t23 = __builtin_amdgcn_perm(u3, u2, 0x00000400u);   // [u2.b0, u3.b0, -, -]
    return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}

// ---------------------------------------------------------------- dequantize
//
// Codes become exact fp16 integers through the bit pattern 0x6400 | u
// (= 1024 + u: the fp16 ulp in [1024, 2048) is 1), the offset is removed
// with an exact packed fma, and q * s16 is one correctly rounded packed fp16
// multiply (fp16 denormals enabled), i.e. exactly fp16_rne(q * s16).

// Pair of 4-bit codes held in one byte (low nibble first) -> (q_lo, q_hi).
// The byte is replicated into bytes 0 and 2; the low nibble stays at bits
// 0..3 (value 1024 + u0) and the high nibble lands at bits 20..23 (value
// 1024 + 16*u1), undone by the 1/16 factor.
__device__ __forceinline__ half2_t q4_pair(uint32_t w, uint32_t sel) {
    uint32_t t = __builtin_amdgcn_perm(w, w, sel);
    t = (t & 0x00F0000Fu) | 0x64006400u;
    const half2_t mul = {(_Float16)1.0f, (_Float16)0.0625f};
    const half2_t add = {(_Float16)-1032.0f, (_Float16)-72.0f};
    return __builtin_elementwise_fma(as_h2(t), mul, add);
}

__device__ __forceinline__ uint4 dequant_q4_chunk(uint32_t w, uint32_t s2) {
    const half2_t s = as_h2(s2);
    uint4 o;
    o.x = as_u32(q4_pair(w, 0x00000000u) * s);
    o.y = as_u32(q4_pair(w, 0x01010101u) * s);
    o.z = as_u32(q4_pair(w, 0x02020202u) * s);
    o.w = as_u32(q4_pair(w, 0x03030303u) * s);
    return o;
}

// Pair of 6-bit codes at bits 0..11 of f -> (q_lo, q_hi).
__device__ __forceinline__ half2_t q6_pair(uint32_t f) {
    uint32_t t = (f & 0x0000FFFFu) | ((f << 10) & 0xFFFF0000u);
    t = (t & 0x003F003Fu) | 0x64006400u;
    const half2_t off = {(_Float16)-1056.0f, (_Float16)-1056.0f};
    return as_h2(t) + off;
}

__device__ __forceinline__ uint4 dequant_q6_chunk(uint32_t lo, uint32_t hi, uint32_t s2) {
    const half2_t s = as_h2(s2);
    uint4 o;
    o.x = as_u32(q6_pair(lo) * s);
    o.y = as_u32(q6_pair(lo >> 12) * s);
    o.z = as_u32(q6_pair(__builtin_amdgcn_alignbit(hi, lo, 24)) * s);
    o.w = as_u32(q6_pair(hi >> 4) * s);
    return o;
}

// Pair of 8-bit codes (bytes SEL0, SEL1 of w) -> fp16 (1024 + u) in each
// half: the byte permute fills the high byte of each half with 0x64.
__device__ __forceinline__ half2_t q8_pair(uint32_t w, uint32_t sel) {
    const uint32_t t = __builtin_amdgcn_perm(0x64646464u, w, sel);
    const half2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    return as_h2(t) + off;
}

__device__ __forceinline__ uint4 dequant_q8_chunk(uint32_t lo, uint32_t hi, uint32_t s2) {
    const half2_t s = as_h2(s2);
    uint4 o;
    o.x = as_u32(q8_pair(lo, 0x04010400u) * s);
    o.y = as_u32(q8_pair(lo, 0x04030402u) * s);
    o.z = as_u32(q8_pair(hi, 0x04010400u) * s);
    o.w = as_u32(q8_pair(hi, 0x04030402u) * s);
    return o;
}

}  // namespace kvq
