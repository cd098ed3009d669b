// kvq_kernels.hip -- gfx950 kernels of the KV-cache format conversions and
// their launchers.
//
// Operations: ExLlamaV2 cache page, Description of fp16_to_fp8 /
// fp8_to_fp16 / fp16_to_q_kv / q_to_fp16_kv (contiguous windows and paged
// caches addressed through block_table / cache_seqlens).
//
// Work decomposition
//   Contiguous 8-bit (the page's fp16_to_fp8 / fp8_to_fp16): each span (one
//     sequence's window) is a contiguous run of width * R elements; threads
//     stream 8-element chunks with 128-bit fp16 and 64-bit byte accesses.
//   K/V conversions (Q4/Q6/Q8, and the per-tensor formats incl. paged
//     8-bit): one wavefront per unit = (token row, tensor, row segment).
//     fp16 -> compact: lane l owns 16 consecutive elements of the segment
//     (1024 elements), so a 32-element block is a lane pair.  compact ->
//     fp16: lane l holds 8-element chunks l and l + 64 of the segment, so
//     each 128-bit store of the wave is contiguous.  The physical row is
//     resolved once per wave from scalar loads of cache_seqlens /
//     block_table.
//
// (The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
// Exllamav2 Ext Cache".)
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

#ifndef KVQ_WAVES_PER_BLOCK
#define KVQ_WAVES_PER_BLOCK 4
#endif
constexpr int kWaves = KVQ_WAVES_PER_BLOCK;   // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------- memory policy
//
// Every conversion streams: its sources (fp16 rows to quantize or narrow,
// codes, scales and bytes to widen back) are loaded, and all of its outputs
// stored, with the non-temporal hint ("nt": streamed through the caches with
// low retention).  A kernel's dirty L2 lines are written back when it ends,
// so outputs that stream out during the kernel shorten its tail.  Measured
// on MI355X at the paged Q4 workload (43 MB per launch, cold rows), against
// ordinary stores: quantize 10.9 -> 10.2 us, dequantize 12.4 -> 11.0 us, and
// a quantize + dequantize step 21.9 -> 21.2 us; the device-scope (sc0/sc1)
// write-through policies were slower per kernel.

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3_t __attribute__((ext_vector_type(3), aligned(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t ld_nt(const uint16_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(uint4* p, uint4 v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st_nt(uint2* p, uint2 v) {
    const u32x2_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}
// 12 bytes at a 4-byte aligned address
__device__ __forceinline__ void st_nt3(void* p, uint32_t a, uint32_t b, uint32_t c) {
    const u32x3_t w = {a, b, c};
    __builtin_nontemporal_store(w, static_cast<u32x3_t*>(p));
}
__device__ __forceinline__ void st_nt(uint16_t* p, uint32_t v) { __builtin_nontemporal_store((uint16_t)v, p); }

// ---------------------------------------------------------------- row map

// Launch geometry, computed by the host launcher for each call.
struct QGeom {
    int32_t n_units;   // rows * ntens * nseg
    int32_t nseg;      // row segments per row
    int32_t ntens;     // tensors present: 1 or 2
    int32_t tens0;     // the tensor when ntens == 1: 0 = K, 1 = V
    FastDiv seq_div;   // logical rows per sequence: width (max_len for kPrefix)
    FastDiv page_div;  // page_size (paged modes)
};

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
    return (__umulhi(n, f.mul) + n) >> f.shift;
}

// How logical rows map to cache rows.
enum RowMode {
    kContig = 0,   // n = b * width + t -> row (b, offset + t)
    kPaged = 1,    // n = b * width + t -> position cache_seqlens[b] + offset + t
    kPrefix = 2,   // n = b * max_len + p -> position p, live while p < cache_seqlens[b] + width
};

// Physical row of logical row n, or -1 when skipped.  Paged positions p live
// in page block_table[b][p / page_size], slot p % page_size, and are skipped
// if p < 0, past the table, or the page is outside [0, dim0).  All values
// are wave-uniform (scalar loads and SALU).  The host bounds n and
// bt_cols * page_size below 2^31, the domain of fast_div.
template <int MODE>
__device__ __forceinline__ int64_t resolve_row(const QLaunch& a, const QGeom& g, int32_t n) {
    const int32_t per_seq = MODE == kPrefix ? a.max_len : a.width;
    const int32_t b = (int32_t)fast_div((uint32_t)n, g.seq_div);
    const int32_t t = n - b * per_seq;
    if (MODE == kContig) return (int64_t)b * a.dim1 + a.offset + t;
    int64_t p;
    if (MODE == kPrefix) {
        p = t;
        if (p >= (int64_t)a.cache_seqlens[b] + a.width) return -1;
    } else {
        p = (int64_t)a.cache_seqlens[b] + a.offset + t;
        if (p < 0) return -1;
    }
    if (p >= (int64_t)a.bt_cols * a.page_size) return -1;
    const uint32_t pu = (uint32_t)p;
    const uint32_t pi = fast_div(pu, g.page_div);
    const int32_t page = a.block_table[(int64_t)b * a.bt_cols + pi];
    if (page < 0 || page >= a.dim0) return -1;
    return (int64_t)page * a.page_size + (int64_t)(pu - pi * (uint32_t)a.page_size);
}

// ---------------------------------------------------------------- work units
//
// A unit is one row segment of one tensor: (logical row n, tensor K or V,
// segment g).  Units are numbered with the segment fastest, then the tensor,
// then the row, so neighbouring waves share the row's paging lookup and
// touch neighbouring memory.  One wavefront converts one unit.

struct UnitRef {
    int64_t row;       // physical row (0 for a padding or skipped unit)
    int32_t tensor;    // 0 = K, 1 = V
    int32_t seg;
    bool live;         // false: nothing to store
};

// Dead units (grid padding past n_units, skipped rows) resolve to row 0 of
// their tensor (always in bounds) with live == false; the kernels return
// at once for them (a wave-uniform branch).
template <int MODE>
__device__ __forceinline__ UnitRef unit_ref(const QLaunch& a, const QGeom& g, int32_t u) {
    UnitRef r;
    r.live = u < g.n_units;
    if (!r.live) u = g.n_units - 1;
    int32_t rt = u;
    r.seg = 0;
    if (g.nseg > 1) {
        rt = u / g.nseg;
        r.seg = u - rt * g.nseg;
    }
    int32_t n;
    if (g.ntens == 2) {
        n = rt >> 1;
        r.tensor = rt & 1;
    } else {
        n = rt;
        r.tensor = g.tens0;
    }
    const int64_t row = resolve_row<MODE>(a, g, n);
    r.live = r.live && row >= 0;
    r.row = row >= 0 ? row : 0;
    return r;
}

__device__ __forceinline__ int32_t wave_index() {
    return (int32_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---------------------------------------------------------------- fp16 -> compact
//
// Lane l of segment g owns the 16 consecutive elements of piece
// pc = 64 g + l (two 128-bit loads); a 32-element block is one lane pair, so
// the block absmax is one DPP exchange.  A segment is 1024 elements; GUARD
// masks the pieces past the row end of a partial last segment (pieces per
// row are even, so a lane pair is in or out together).

// Pieces past the row end (in == false) read nothing and yield zeros.
__device__ __forceinline__ void load_piece(const QLaunch& a, const UnitRef& ur, int32_t pc, bool in,
                                           uint4& x0, uint4& x1) {
    const uint4* src = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(ur.tensor ? a.v_src : a.k_src) + ur.row * a.R) + 2 * pc;
    x0 = make_uint4(0, 0, 0, 0);
    x1 = make_uint4(0, 0, 0, 0);
    if (in) {
        x0 = ld_nt(src);
        x1 = ld_nt(src + 1);
    }
}

// Block quantization of one unit.
template <int WBITS, bool GUARD>
__device__ __forceinline__ void quant_unit(const QLaunch& a, const UnitRef& ur, int lane) {
    const int32_t R = a.R;
    const int32_t pc = ur.seg * 64 + lane;
    const bool in = !GUARD || pc < (R >> 4);
    uint4 x0, x1;
    load_piece(a, ur, pc, in, x0, x1);
    const uint32_t s16 = scale_from_absmax<WBITS>(pair_max(absmax_2chunks(x0, x1)));
    const ScaleOps so = prep_scale(s16);
    uint32_t u0[8], u1[8];
    quant_chunk<WBITS>(x0, s16, so, u0);
    quant_chunk<WBITS>(x1, s16, so, u1);

    const bool store = ur.live && in;
    uint8_t* codes = static_cast<uint8_t*>(ur.tensor ? a.v_dst : a.k_dst) + ur.row * (int64_t)(R / 8 * WBITS);
    if constexpr (WBITS == 4) {
        const uint2 d = make_uint2(pack_q4(u0), pack_q4(u1));
        if (store) st_nt(reinterpret_cast<uint2*>(codes + 8 * pc), d);
    } else if constexpr (WBITS == 8) {
        const uint4 d = make_uint4(pack_q8x4(u0[0], u0[1], u0[2], u0[3]), pack_q8x4(u0[4], u0[5], u0[6], u0[7]),
                                   pack_q8x4(u1[0], u1[1], u1[2], u1[3]), pack_q8x4(u1[4], u1[5], u1[6], u1[7]));
        if (store) st_nt(reinterpret_cast<uint4*>(codes + 16 * pc), d);
    } else {
        uint32_t lo0, hi0, lo1, hi1;
        pack_q6(u0, lo0, hi0);
        pack_q6(u1, lo1, hi1);
        const uint32_t d1 = __builtin_amdgcn_perm(lo1, hi0, 0x05040100u);   // hi0.lo16 | lo1.lo16 << 16
        const uint32_t d2 = __builtin_amdgcn_alignbit(hi1, lo1, 16);        // lo1 >> 16 | hi1 << 16
        if (store) st_nt3(codes + 12 * pc, lo0, d1, d2);
    }
    uint16_t* scales = static_cast<uint16_t*>(ur.tensor ? a.v_scales : a.k_scales) + ur.row * (int64_t)(R >> 5);
    if (store && (lane & 1) == 0) st_nt(scales + (pc >> 1), s16);
}

// high byte of each fp16: bytes 1,3 of the first word then 1,3 of the second
__device__ __forceinline__ uint32_t high_bytes(uint32_t w0, uint32_t w1) {
    return __builtin_amdgcn_perm(w1, w0, 0x07050301u);
}

// 8-bit (high byte) narrowing of one unit: 16 bytes per lane.
template <bool GUARD>
__device__ __forceinline__ void narrow_unit(const QLaunch& a, const UnitRef& ur, int lane) {
    const int32_t pc = ur.seg * 64 + lane;
    const bool in = !GUARD || pc < (a.R >> 4);
    uint4 x0, x1;
    load_piece(a, ur, pc, in, x0, x1);
    const uint4 d = make_uint4(high_bytes(x0.x, x0.y), high_bytes(x0.z, x0.w),
                               high_bytes(x1.x, x1.y), high_bytes(x1.z, x1.w));
    uint8_t* out = static_cast<uint8_t*>(ur.tensor ? a.v_dst : a.k_dst) + ur.row * (int64_t)a.R;
    if (ur.live && in) st_nt(reinterpret_cast<uint4*>(out + 16 * pc), d);
}

template <int WBITS, int MODE, bool GUARD>
__global__ __launch_bounds__(kThreads) void quant_kv_kernel(QLaunch a, QGeom g) {
    const UnitRef ur = unit_ref<MODE>(a, g, wave_index());
    if (!ur.live) return;   // wave-uniform: skipped rows and grid padding do nothing
    quant_unit<WBITS, GUARD>(a, ur, threadIdx.x & 63);
}

// Per-tensor formats: the unit's tensor picks its format (wave-uniform).
template <int MODE, bool GUARD>
__global__ __launch_bounds__(kThreads) void narrow_kv_kernel(QLaunch a, QGeom g) {
    const UnitRef ur = unit_ref<MODE>(a, g, wave_index());
    if (!ur.live) return;   // wave-uniform: skipped rows and grid padding do nothing
    const int lane = threadIdx.x & 63;
    switch (ur.tensor ? a.fmt_v : a.fmt_k) {
        case 4: quant_unit<4, GUARD>(a, ur, lane); break;
        case 6: quant_unit<6, GUARD>(a, ur, lane); break;
        case 8: quant_unit<8, GUARD>(a, ur, lane); break;
        default: narrow_unit<GUARD>(a, ur, lane); break;
    }
}

// ---------------------------------------------------------------- compact -> fp16
//
// Lane l holds chunks (8 elements) c = NCH * 64 g + 64 k + l, k < NCH, so
// every 128-bit store of the wave is contiguous.

struct CodeChunk {
    uint32_t lo, hi;    // Q4: lo = 8 codes; Q6: the 8 bytes holding the 6 code bytes; Q8: 8 codes
    uint32_t s;         // scale (fp16 bits)
};

template <int WBITS>
__device__ __forceinline__ CodeChunk load_code_chunk(const uint8_t* __restrict__ codes_row,
                                                     const uint16_t* __restrict__ scales_row,
                                                     int32_t c) {
    CodeChunk q;
    if constexpr (WBITS == 4) {
        q.lo = ld_nt(reinterpret_cast<const uint32_t*>(codes_row) + c);
        q.hi = 0;
    } else if constexpr (WBITS == 8) {
        const uint32_t* g = reinterpret_cast<const uint32_t*>(codes_row) + 2 * c;
        q.lo = ld_nt(g);
        q.hi = ld_nt(g + 1);
    } else {
        // chunk c's 6 bytes start at 6c: load the 8 bytes of its 12-byte
        // group that contain them (4-byte aligned); odd chunks are shifted
        // into place after the load.
        const uint32_t* g = reinterpret_cast<const uint32_t*>(codes_row + 12 * (c >> 1) + 4 * (c & 1));
        q.lo = ld_nt(g);
        q.hi = ld_nt(g + 1);
    }
    q.s = ld_nt(scales_row + (c >> 2));
    return q;
}

// The codes of chunk c only (the caller supplies q.s).
template <int WBITS>
__device__ __forceinline__ CodeChunk load_code_only(const uint8_t* __restrict__ codes_row, int32_t c) {
    CodeChunk q;
    if constexpr (WBITS == 4) {
        q.lo = ld_nt(reinterpret_cast<const uint32_t*>(codes_row) + c);
        q.hi = 0;
    } else if constexpr (WBITS == 8) {
        const uint32_t* g = reinterpret_cast<const uint32_t*>(codes_row) + 2 * c;
        q.lo = ld_nt(g);
        q.hi = ld_nt(g + 1);
    } else {
        const uint32_t* g = reinterpret_cast<const uint32_t*>(codes_row + 12 * (c >> 1) + 4 * (c & 1));
        q.lo = ld_nt(g);
        q.hi = ld_nt(g + 1);
    }
    q.s = 0;
    return q;
}

template <int WBITS>
__device__ __forceinline__ uint4 dequant_chunk(const CodeChunk& q, int32_t c) {
    const uint32_t s2 = q.s | (q.s << 16);
    if constexpr (WBITS == 4) {
        return dequant_q4_chunk(q.lo, s2);
    } else if constexpr (WBITS == 8) {
        return dequant_q8_chunk(q.lo, q.hi, s2);
    } else {
        uint32_t lo, hi;
        if (c & 1) {
            lo = __builtin_amdgcn_alignbit(q.hi, q.lo, 16);
            hi = q.hi >> 16;
        } else {
            lo = q.lo;
            hi = q.hi & 0xFFFFu;
        }
        return dequant_q6_chunk(lo, hi, s2);
    }
}

// Block dequantization of one unit.  SSCALE: fetch the segment's scales
// with one scalar load instead of per-lane loads (whole segments only).
// Measured within one build at the paged workload (43 MB per launch): the
// single-width Q4 kernel -2% and Q8 -5%, Q6 unchanged, and the per-tensor
// kernel (format switch) +6%; so only the single-width Q4 and Q8 kernels
// enable it.
template <int WBITS, int NCH, bool GUARD, bool SSCALE>
__device__ __forceinline__ void dequant_unit(const QLaunch& a, const UnitRef& ur, int lane) {
    const int32_t R = a.R;
    const int32_t cpr = R >> 3;
    const uint8_t* codes = static_cast<const uint8_t*>(ur.tensor ? a.v_src : a.k_src) +
                           ur.row * (int64_t)(R / 8 * WBITS);
    const uint16_t* scales = static_cast<const uint16_t*>(ur.tensor ? a.v_scales : a.k_scales) +
                             ur.row * (int64_t)(R >> 5);
    CodeChunk q[NCH];
    if constexpr (GUARD || !SSCALE) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int32_t c = ur.seg * (NCH * 64) + k * 64 + lane;
            if (GUARD) q[k] = c < cpr ? load_code_chunk<WBITS>(codes, scales, c) : CodeChunk{0, 0, 0};
            else q[k] = load_code_chunk<WBITS>(codes, scales, c);
        }
    } else {
        // Whole segment: its NCH * 16 scales are NCH * 8 dwords inside the
        // row, 32-byte aligned (R is a multiple of 512 here), fetched with one
        // scalar load; lane l picks the scale of its chunks k * 64 + l (block
        // (k * 64 + l) / 4: dword k * 8 + l / 8, half (l / 4) & 1).
        const uint32_t* sw = reinterpret_cast<const uint32_t*>(scales) + ur.seg * (NCH * 8);
        uint32_t S[NCH * 8];
#pragma unroll
        for (int i = 0; i < NCH * 8; ++i) S[i] = __builtin_amdgcn_readfirstlane(sw[i]);
        const int32_t di = lane >> 3;
        const bool hi = (lane >> 2) & 1;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int32_t c = ur.seg * (NCH * 64) + k * 64 + lane;
            q[k] = load_code_only<WBITS>(codes, c);
            uint32_t w = S[k * 8];
#pragma unroll
            for (int i = 1; i < 8; ++i) w = di == i ? S[k * 8 + i] : w;
            q[k].s = hi ? (w >> 16) : (w & 0xFFFFu);
        }
    }
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(ur.tensor ? a.v_dst : a.k_dst) + ur.row * R);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int32_t c = ur.seg * (NCH * 64) + k * 64 + lane;
        const uint4 o = dequant_chunk<WBITS>(q[k], c);
        if (ur.live && (!GUARD || c < cpr)) st_nt(dst + c, o);
    }
}

// bytes 0,1 of w -> fp16 patterns byte << 8 in the low and high halves
__device__ __forceinline__ uint32_t widen_lo(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x01040004u); }
__device__ __forceinline__ uint32_t widen_hi(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x03040204u); }

// 8-bit (high byte) widening of one unit.
template <int NCH, bool GUARD>
__device__ __forceinline__ void widen_unit(const QLaunch& a, const UnitRef& ur, int lane) {
    const int32_t R = a.R;
    const int32_t cpr = R >> 3;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(
        static_cast<const uint8_t*>(ur.tensor ? a.v_src : a.k_src) + ur.row * (int64_t)R);
    uint2 v[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int32_t c = ur.seg * (NCH * 64) + k * 64 + lane;
        v[k] = make_uint2(0, 0);
        if (!GUARD || c < cpr) v[k] = make_uint2(ld_nt(src + 2 * c), ld_nt(src + 2 * c + 1));
    }
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(ur.tensor ? a.v_dst : a.k_dst) + ur.row * R);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int32_t c = ur.seg * (NCH * 64) + k * 64 + lane;
        const uint4 o = make_uint4(widen_lo(v[k].x), widen_hi(v[k].x), widen_lo(v[k].y), widen_hi(v[k].y));
        if (ur.live && (!GUARD || c < cpr)) st_nt(dst + c, o);
    }
}

template <int WBITS, int MODE, int NCH, bool GUARD>
__global__ __launch_bounds__(kThreads) void dequant_kv_kernel(QLaunch a, QGeom g) {
    const UnitRef ur = unit_ref<MODE>(a, g, wave_index());
    if (!ur.live) return;   // wave-uniform: skipped rows and grid padding do nothing
    dequant_unit<WBITS, NCH, GUARD, WBITS != 6>(a, ur, threadIdx.x & 63);
}

template <int MODE, int NCH, bool GUARD>
__global__ __launch_bounds__(kThreads) void widen_kv_kernel(QLaunch a, QGeom g) {
    const UnitRef ur = unit_ref<MODE>(a, g, wave_index());
    if (!ur.live) return;   // wave-uniform: skipped rows and grid padding do nothing
    const int lane = threadIdx.x & 63;
    switch (ur.tensor ? a.fmt_v : a.fmt_k) {
        case 4: dequant_unit<4, NCH, GUARD, false>(a, ur, lane); break;
        case 6: dequant_unit<6, NCH, GUARD, false>(a, ur, lane); break;
        case 8: dequant_unit<8, NCH, GUARD, false>(a, ur, lane); break;
        default: widen_unit<NCH, GUARD>(a, ur, lane); break;
    }
}

// ---------------------------------------------------------------- 8-bit

// Contiguous windows: each sequence's window is one run of width * R
// elements, streamed 8 elements per chunk, CPT chunks per thread (4 for
// large spans; 1 when that would leave the grid smaller than the chip).
template <int CPT>
__global__ __launch_bounds__(kThreads) void fp16_to_fp8_kernel(Fp8Launch a) {
    const int64_t cps = a.span_elems >> 3;
    const int64_t c0 = (int64_t)blockIdx.x * (kThreads * CPT) + threadIdx.x;
    for (int32_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const int64_t e0 = (int64_t)b * a.batch_stride_elems + a.first_elem;
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.in) + e0);
        uint2* dst = reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.out) + e0);
        uint4 v[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t c = c0 + k * kThreads;
            v[k] = c < cps ? ld_nt(src + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t c = c0 + k * kThreads;
            if (c < cps) st_nt(dst + c, make_uint2(high_bytes(v[k].x, v[k].y), high_bytes(v[k].z, v[k].w)));
        }
    }
}

template <int CPT>
__global__ __launch_bounds__(kThreads) void fp8_to_fp16_kernel(Fp8Launch a) {
    const int64_t cps = a.span_elems >> 3;
    const int64_t c0 = (int64_t)blockIdx.x * (kThreads * CPT) + threadIdx.x;
    for (int32_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const int64_t e0 = (int64_t)b * a.batch_stride_elems + a.first_elem;
        const uint2* src = reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a.in) + e0);
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + e0);
        uint2 v[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t c = c0 + k * kThreads;
            v[k] = c < cps ? make_uint2(ld_nt(reinterpret_cast<const uint32_t*>(src + c)),
                                        ld_nt(reinterpret_cast<const uint32_t*>(src + c) + 1))
                           : make_uint2(0, 0);
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t c = c0 + k * kThreads;
            if (c < cps)
                st_nt(dst + c, make_uint4(widen_lo(v[k].x), widen_hi(v[k].x), widen_lo(v[k].y), widen_hi(v[k].y)));
        }
    }
}

// ---------------------------------------------------------------- self-test kernels

// u[i * nx + j] = code of x[j] under scale s[i], through the same routines
// as quant_kv_kernel (one thread per chunk of 8 x values).  CLAMP_ALL forces
// the clamping path; otherwise the kernels' dispatch on the scale is used.
template <int WBITS, bool CLAMP_ALL>
__global__ __launch_bounds__(kThreads) void selftest_codes_kernel(const uint16_t* __restrict__ x, int64_t nx,
                                                                  const uint16_t* __restrict__ s16,
                                                                  int64_t ns, uint8_t* __restrict__ u) {
    const int64_t cpr = nx >> 3;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= cpr * ns) return;
    const int64_t i = t / cpr, j = t - i * cpr;
    const uint4 v = reinterpret_cast<const uint4*>(x)[j];
    const uint32_t s = s16[i];
    const ScaleOps so = prep_scale(s);
    uint32_t c[8];
    if (CLAMP_ALL) quant_chunk_clamped<WBITS>(v, so, c);
    else quant_chunk<WBITS>(v, s, so, c);
    constexpr uint32_t mask = (1u << WBITS) - 1;
    uint2 o;
    o.x = (c[0] & mask) | ((c[1] & mask) << 8) | ((c[2] & mask) << 16) | ((c[3] & mask) << 24);
    o.y = (c[4] & mask) | ((c[5] & mask) << 8) | ((c[6] & mask) << 16) | ((c[7] & mask) << 24);
    reinterpret_cast<uint2*>(u + i * nx)[j] = o;
}

template <int WBITS>
__global__ __launch_bounds__(kThreads) void selftest_scales_kernel(const uint16_t* __restrict__ a, int64_t n,
                                                                   uint16_t* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t < n) out[t] = (uint16_t)scale_from_absmax<WBITS>(a[t]);
}

__global__ __launch_bounds__(kThreads) void selftest_fastdiv_kernel(const uint32_t* __restrict__ n, int64_t count,
                                                                      FastDiv f, uint32_t* __restrict__ q) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t < count) q[t] = fast_div(n[t], f);
}

// ---------------------------------------------------------------- launchers

static int launch(const void* fn, dim3 grid, dim3 block, void** args, void* stream) {
    return (int)hipLaunchKernel(fn, grid, block, args, 0, static_cast<hipStream_t>(stream));
}

// Chunks per thread: 4 unless the grid would then have fewer workgroups
// than the chip has CUs (small windows), where 1 spreads the span wider.
static int fp8_cpt(const Fp8Launch& a) {
    const int64_t cps = a.span_elems >> 3;
    const int64_t blocks4 = (cps + kThreads * 4 - 1) / (kThreads * 4) * (int64_t)a.batch;
    return blocks4 < 256 ? 1 : 4;
}

static dim3 fp8_grid(const Fp8Launch& a, int cpt) {
    const int64_t cps = a.span_elems >> 3;
    const int64_t gx = (cps + kThreads * cpt - 1) / (kThreads * cpt);
    const int32_t gy = a.batch < 65535 ? a.batch : 65535;
    return dim3((unsigned)gx, (unsigned)gy, 1);
}

int launch_fp16_to_fp8(const Fp8Launch& a, void* stream) {
    Fp8Launch arg = a;
    void* args[] = {&arg};
    const int cpt = fp8_cpt(a);
    const void* fn = cpt == 1 ? reinterpret_cast<const void*>(&fp16_to_fp8_kernel<1>)
                              : reinterpret_cast<const void*>(&fp16_to_fp8_kernel<4>);
    return launch(fn, fp8_grid(a, cpt), dim3(kThreads), args, stream);
}

int launch_fp8_to_fp16(const Fp8Launch& a, void* stream) {
    Fp8Launch arg = a;
    void* args[] = {&arg};
    const int cpt = fp8_cpt(a);
    const void* fn = cpt == 1 ? reinterpret_cast<const void*>(&fp8_to_fp16_kernel<1>)
                              : reinterpret_cast<const void*>(&fp8_to_fp16_kernel<4>);
    return launch(fn, fp8_grid(a, cpt), dim3(kThreads), args, stream);
}

// Kernel variants.  fp16 -> compact: 64 lanes x 16 elements per segment,
// guarded when the row's 16-element pieces are not a multiple of 64.
// compact -> fp16: NCH chunks of 8 per lane, NCH = 2 (or 1) when the row's
// chunks are a multiple of 128 (or 64), else NCH = 2 guarded.  The
// single-format kernels serve the page's one-wbits calls; the per-tensor
// kernels pick each unit's format at run time.
template <int W, int MODE>
static const void* quant_fn(bool guard) {
    return guard ? reinterpret_cast<const void*>(&quant_kv_kernel<W, MODE, true>)
                 : reinterpret_cast<const void*>(&quant_kv_kernel<W, MODE, false>);
}

template <int MODE>
static const void* narrow_fn(bool guard) {
    return guard ? reinterpret_cast<const void*>(&narrow_kv_kernel<MODE, true>)
                 : reinterpret_cast<const void*>(&narrow_kv_kernel<MODE, false>);
}

template <int W, int MODE>
static const void* dequant_fn(int nch, bool guard) {
    if (guard) return reinterpret_cast<const void*>(&dequant_kv_kernel<W, MODE, 2, true>);
    if (nch == 2) return reinterpret_cast<const void*>(&dequant_kv_kernel<W, MODE, 2, false>);
    return reinterpret_cast<const void*>(&dequant_kv_kernel<W, MODE, 1, false>);
}

template <int MODE>
static const void* widen_fn(int nch, bool guard) {
    if (guard) return reinterpret_cast<const void*>(&widen_kv_kernel<MODE, 2, true>);
    if (nch == 2) return reinterpret_cast<const void*>(&widen_kv_kernel<MODE, 2, false>);
    return reinterpret_cast<const void*>(&widen_kv_kernel<MODE, 1, false>);
}

template <int W>
static const void* single_fn(bool to_compact, int mode, int nch, bool guard) {
    if (to_compact) return mode == kPaged ? quant_fn<W, kPaged>(guard) : quant_fn<W, kContig>(guard);
    if (mode == kPrefix) return dequant_fn<W, kPrefix>(nch, guard);
    return mode == kPaged ? dequant_fn<W, kPaged>(nch, guard) : dequant_fn<W, kContig>(nch, guard);
}

static const void* mixed_fn(bool to_compact, int mode, int nch, bool guard) {
    if (to_compact) return mode == kPaged ? narrow_fn<kPaged>(guard) : narrow_fn<kContig>(guard);
    if (mode == kPrefix) return widen_fn<kPrefix>(nch, guard);
    return mode == kPaged ? widen_fn<kPaged>(nch, guard) : widen_fn<kContig>(nch, guard);
}

// mixed: per-tensor formats (a.fmt_k / a.fmt_v); otherwise one width a.wbits
static int launch_units(const QLaunch& a, bool to_compact, bool mixed, int mode, void* stream) {
    int nch = 2;
    bool guard = false;
    int32_t seg_elems;
    if (to_compact) {
        guard = (a.R / 16) % 64 != 0;
        seg_elems = 1024;
    } else {
        const int32_t cpr = a.R >> 3;
        if (cpr % 128 == 0) nch = 2;
        else if (cpr % 64 == 0) nch = 1;
        else guard = true;
        seg_elems = nch * 64 * 8;
    }
    const int64_t rows = (int64_t)a.batch * (mode == kPrefix ? a.max_len : a.width);
    QGeom g;
    g.nseg = (a.R + seg_elems - 1) / seg_elems;
    g.ntens = (a.k_src ? 1 : 0) + (a.v_src ? 1 : 0);
    g.tens0 = a.k_src ? 0 : 1;
    g.n_units = (int32_t)(rows * g.ntens * g.nseg);   // bounded by the host checks
    g.seq_div = make_fastdiv((uint32_t)(mode == kPrefix ? a.max_len : a.width));
    g.page_div = make_fastdiv(a.page_size > 0 ? (uint32_t)a.page_size : 1u);
    const dim3 grid((unsigned)((g.n_units + kWaves - 1) / kWaves));
    QLaunch arg = a;
    void* args[] = {&arg, &g};
    // Per-tensor widening where every present tensor is Q4 (or every one
    // Q8) runs the single-width kernel of that width: it has the scalar
    // scale fetch, which the format-switch kernel does not take.
    int wbits = a.wbits;
    if (mixed && !to_compact) {
        const int fk = a.k_src ? a.fmt_k : -1, fv = a.v_src ? a.fmt_v : -1;
        const int f = fk < 0 ? fv : (fv < 0 || fv == fk ? fk : -1);
        if (f == 4 || f == 8) {
            mixed = false;
            wbits = f;
        }
    }
    const void* fn;
    if (mixed) fn = mixed_fn(to_compact, mode, nch, guard);
    else if (wbits == 4) fn = single_fn<4>(to_compact, mode, nch, guard);
    else if (wbits == 6) fn = single_fn<6>(to_compact, mode, nch, guard);
    else fn = single_fn<8>(to_compact, mode, nch, guard);
    return launch(fn, grid, dim3(kThreads), args, stream);
}

int launch_quant_kv(const QLaunch& a, void* stream) {
    return launch_units(a, true, false, a.page_size ? kPaged : kContig, stream);
}

int launch_dequant_kv(const QLaunch& a, void* stream) {
    return launch_units(a, false, false, a.page_size ? kPaged : kContig, stream);
}

int launch_fp16_to_kv(const QLaunch& a, void* stream) {
    return launch_units(a, true, true, a.page_size ? kPaged : kContig, stream);
}

int launch_kv_to_fp16(const QLaunch& a, void* stream) {
    return launch_units(a, false, true, a.page_size ? kPaged : kContig, stream);
}

int launch_kv_to_fp16_prefix(const QLaunch& a, void* stream) {
    return launch_units(a, false, true, kPrefix, stream);
}

int launch_selftest_codes(const uint16_t* x, int64_t nx, const uint16_t* s, int64_t ns, int wbits,
                          bool force_clamp, uint8_t* u, void* stream) {
    const int64_t threads = (nx >> 3) * ns;
    dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    void* args[] = {&x, &nx, &s, &ns, &u};
    const void* fn;
    if (wbits == 4)
        fn = force_clamp ? reinterpret_cast<const void*>(&selftest_codes_kernel<4, true>)
                         : reinterpret_cast<const void*>(&selftest_codes_kernel<4, false>);
    else if (wbits == 6)
        fn = force_clamp ? reinterpret_cast<const void*>(&selftest_codes_kernel<6, true>)
                         : reinterpret_cast<const void*>(&selftest_codes_kernel<6, false>);
    else
        fn = force_clamp ? reinterpret_cast<const void*>(&selftest_codes_kernel<8, true>)
                         : reinterpret_cast<const void*>(&selftest_codes_kernel<8, false>);
    return launch(fn, grid, dim3(kThreads), args, stream);
}

int launch_selftest_scales(const uint16_t* a, int64_t n, int wbits, uint16_t* out, void* stream) {
    dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    void* args[] = {&a, &n, &out};
    const void* fn = wbits == 4 ? reinterpret_cast<const void*>(&selftest_scales_kernel<4>)
                   : wbits == 6 ? reinterpret_cast<const void*>(&selftest_scales_kernel<6>)
                                : reinterpret_cast<const void*>(&selftest_scales_kernel<8>);
    return launch(fn, grid, dim3(kThreads), args, stream);
}

int launch_selftest_fastdiv(const uint32_t* n, int64_t count, uint32_t d, uint32_t* q, void* stream) {
    FastDiv f = make_fastdiv(d);
    dim3 grid((unsigned)((count + kThreads - 1) / kThreads));
    void* args[] = {&n, &count, &f, &q};
    return launch(reinterpret_cast<const void*>(&selftest_fastdiv_kernel), grid, dim3(kThreads), args, stream);
}

}  // namespace kvq
