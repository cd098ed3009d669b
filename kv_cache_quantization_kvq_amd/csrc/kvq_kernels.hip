// kvq_kernels.hip -- gfx950 kernels of the KV-cache format conversions and
// their launchers.
//
// Operations: ExLlamaV2 cache page, Description of fp16_to_fp8 /
// fp8_to_fp16 / fp16_to_q_kv / q_to_fp16_kv (contiguous windows and paged
// caches addressed through block_table / cache_seqlens).
//
// Work decomposition
//   A "unit" is one 1024-element segment of one token row of one tensor
//   (K or V); rows whose length R is not a multiple of 1024 end in a partial
//   segment.  Token rows are (sequence b, position t < width) for the
//   page's calls, or (b, position p < max_len) for the full-prefix widen.
//
//   fp16 -> compact (quantize, 8-bit narrow), R % 1024 == 0: one wavefront
//     per pair of units of one tensor, in that tensor's format when K and
//     V formats differ.  The wave reads its 4 KB of fp16 with
//     contiguous 16-byte lanes, passes it through LDS, and lane L then owns
//     32-element block L (unit L / 32): the absmax, scale and codes of a
//     block are one lane's work.  Q4 codes (16 bytes per block) are stored
//     straight from the lane; Q6 / Q8 codes are restaged through LDS so
//     every store is 16 contiguous bytes per lane.  8-bit narrowing needs no
//     transpose.  Every paged Q6 / Q8 launch, and any launch of one block
//     format up to 4,096 units, instead takes one wavefront per unit: two
//     whole 1 KB loads, an LDS pass that hands lane l elements 16 l ..
//     16 l + 15, a block per lane pair, codes stored straight from each
//     lane (8, 12 or 16 contiguous bytes).
//   fp16 -> compact, other R: one wavefront per unit, lane l holding 16
//     consecutive elements (a block is a lane pair).
//   compact -> fp16 (dequantize, 8-bit widen, full-prefix widen): one
//     wavefront per run of P consecutive positions of one sequence (P = 1,
//     2, 4 or 8 by launch size), both tensors (or one tensor when K and V
//     formats differ, or for large contiguous launches).  Every load of
//     the wave is issued before its first store, and the stores go tensor
//     by tensor; lane l converts chunks (8 elements) l and l + 64 of each
//     unit, so every 128-bit store of the wave is contiguous.
//   The paged row of a position is resolved from scalar loads of
//   cache_seqlens[b] and block_table[b][p / page_size], once per run.
//
// (The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
// Exllamav2 Ext Cache".)
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kWaves = 4;                 // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------- memory policy
//
// Every conversion streams: its sources (fp16 rows to quantize or narrow,
// codes, scales and bytes to widen back) are loaded, and all of its outputs
// stored, with the non-temporal hint ("nt": streamed through the caches with
// low retention).  A kernel's dirty L2 lines are written back when it ends,
// so outputs that stream out during the kernel shorten its tail.

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3_t __attribute__((ext_vector_type(3), aligned(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
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
__device__ __forceinline__ void st_nt(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
// 12 bytes at a 4-byte aligned address
__device__ __forceinline__ void st_nt3(void* p, uint32_t a, uint32_t b, uint32_t c) {
    const u32x3_t w = {a, b, c};
    __builtin_nontemporal_store(w, static_cast<u32x3_t*>(p));
}
__device__ __forceinline__ void st_nt(uint16_t* p, uint32_t v) { __builtin_nontemporal_store((uint16_t)v, p); }

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
    return (__umulhi(n, f.mul) + n) >> f.shift;
}

// How positions map to cache rows.
enum RowMode {
    kContig = 0,   // position t of sequence b -> row (b, offset + t)
    kPaged = 1,    // position t of sequence b -> cache position cache_seqlens[b] + offset + t
    kPrefix = 2,   // position p of sequence b, live while p < cache_seqlens[b] + width
};

// Cache rows of NP positions t0 + d[k] of sequence b (d[k] in [0, NP); tin[k]
// false: no position), or -1 when skipped.  Paged positions p live in page
// block_table[b][p / page_size], slot p % page_size, and are skipped if
// p < 0, past the table, or the page is outside [0, dim0).  All values are
// wave-uniform (scalar loads and SALU).  The first position is clamped into
// [-NP, lim] once (lim = bt_cols * page_size <= 2^30, a host bound), so
// every per-position test is 32-bit and branch-free, and the block-table
// loads of all NP positions issue together after the one load of
// cache_seqlens[b].
template <int MODE, int NP>
__device__ __forceinline__ void resolve_positions(const QLaunch& a, FastDiv page_div, int32_t b, int32_t t0,
                                                  const int32_t (&d)[NP], const bool (&tin)[NP],
                                                  int64_t (&row)[NP]) {
    if constexpr (MODE == kContig) {
        const int64_t r0 = (int64_t)b * a.dim1 + a.offset + t0;
#pragma unroll
        for (int k = 0; k < NP; ++k) row[k] = tin[k] ? r0 + d[k] : -1;
    } else {
        const int32_t sl = a.cache_seqlens[b];
        const int32_t lim = a.bt_cols * a.page_size;
        // prefix: positions from 0, live below cache_seqlens[b] + width
        const int64_t p0l = (MODE == kPrefix ? 0 : (int64_t)sl + a.offset) + t0;
        const int32_t p0 = (int32_t)(p0l < -NP ? -NP : (p0l > lim ? lim : p0l));
        int32_t end = lim;
        if (MODE == kPrefix) {
            const int64_t e = (int64_t)sl + a.width;
            end = (int32_t)(e < 0 ? 0 : (e > lim ? lim : e));
        }
        const int32_t* bt = a.block_table + (int64_t)b * a.bt_cols;
        uint32_t pu[NP], pi[NP];
        int32_t page[NP];
        bool ok[NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int32_t p = p0 + d[k];
            ok[k] = tin[k] & (p >= 0) & (p < end);
            pu[k] = ok[k] ? (uint32_t)p : 0u;
            pi[k] = fast_div(pu[k], page_div);
            page[k] = bt[pi[k]];            // entry 0 for a skipped position (bt_cols >= 1)
        }
        // every entry is used whatever ok[k] says, so no load moves under a
        // branch (each would then wait before the next issued)
#pragma unroll
        for (int k = 0; k < NP; ++k) page[k] = __builtin_amdgcn_readfirstlane(page[k]);
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const bool live = ok[k] & ((uint32_t)page[k] < (uint32_t)a.dim0);
            row[k] = live ? (int64_t)page[k] * a.page_size + (int64_t)(pu[k] - pi[k] * (uint32_t)a.page_size) : -1;
        }
    }
}

// ================================================================ one unit per wave
//
// fp16 -> compact for rows whose length is not a multiple of 1024.  A unit
// is (logical row n, tensor, segment g), numbered with the segment fastest,
// then the tensor, then the row.  Lane l of segment g owns the 16
// consecutive elements of piece pc = 64 g + l (two 128-bit loads); a
// 32-element block is one lane pair, so the block absmax is one DPP
// exchange.  GUARD masks the pieces past the row end of a partial last
// segment (pieces per row are even, so a lane pair is in or out together).

struct QGeom {
    int32_t n_units;   // rows * ntens * nseg
    int32_t nseg;      // row segments per row
    int32_t ntens;     // tensors present: 1 or 2
    int32_t tens0;     // the tensor when ntens == 1: 0 = K, 1 = V
    FastDiv seq_div;   // logical rows per sequence: width
    FastDiv page_div;  // page_size (paged modes)
};

struct UnitRef {
    int64_t row;       // physical row (0 for a padding or skipped unit)
    int32_t tensor;    // 0 = K, 1 = V
    int32_t seg;
    bool live;         // false: nothing to store
};

// Dead units (grid padding past n_units, skipped rows) resolve to row 0 of
// their tensor (always in bounds) with live == false.
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
    const int32_t b = (int32_t)fast_div((uint32_t)n, g.seq_div);
    const int32_t d[1] = {0};
    const bool tin[1] = {true};
    int64_t row[1];
    resolve_positions<MODE, 1>(a, g.page_div, b, n - b * a.width, d, tin, row);
    r.live = r.live && row[0] >= 0;
    r.row = row[0] >= 0 ? row[0] : 0;
    return r;
}

__device__ __forceinline__ int32_t wave_index() {
    return (int32_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

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

template <int WBITS, bool GUARD>
__device__ __forceinline__ void quant_unit(const QLaunch& a, const UnitRef& ur, int lane) {
    const int32_t R = a.R;
    const int32_t pc = ur.seg * 64 + lane;
    const bool in = !GUARD || pc < (R >> 4);
    uint4 x0, x1;
    load_piece(a, ur, pc, in, x0, x1);
    const uint32_t s16 = scale_from_absmax<WBITS>(pair_max(absmax_2chunks(x0, x1)));
    const ScaleOps so = prep_scale(s16);
    const uint4 x[2] = {x0, x1};
    uint32_t u[2][8];
    quant_chunks<WBITS, 2>(x, s16, so, u);
    const uint32_t (&u0)[8] = u[0];
    const uint32_t (&u1)[8] = u[1];

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
__global__ __launch_bounds__(kThreads) void quant_unit_kernel(QLaunch a, QGeom g) {
    const UnitRef ur = unit_ref<MODE>(a, g, wave_index());
    if (!ur.live) return;   // wave-uniform: skipped rows and grid padding do nothing
    quant_unit<WBITS, GUARD>(a, ur, threadIdx.x & 63);
}

// Per-tensor formats: the unit's tensor picks its format (wave-uniform).
template <int MODE, bool GUARD>
__global__ __launch_bounds__(kThreads) void narrow_unit_kernel(QLaunch a, QGeom g) {
    const UnitRef ur = unit_ref<MODE>(a, g, wave_index());
    if (!ur.live) return;
    const int lane = threadIdx.x & 63;
    switch (ur.tensor ? a.fmt_v : a.fmt_k) {
        case 4: quant_unit<4, GUARD>(a, ur, lane); break;
        case 6: quant_unit<6, GUARD>(a, ur, lane); break;
        case 8: quant_unit<8, GUARD>(a, ur, lane); break;
        default: narrow_unit<GUARD>(a, ur, lane); break;
    }
}

// ================================================================ wave-group geometry
//
// Workgroups are dealt round-robin to the chip's 8 XCDs (each with its own
// L2).  With XCD set, workgroup ids are renumbered so that each XCD takes one
// contiguous range of groups: the waves sharing a sequence -- and its
// cache_seqlens and block_table lines -- then share one L2.  The renumbering
// is a bijection of [0, grid) for grids that are a multiple of 8 (the
// launcher pads the grid).

struct GroupGeom {
    int32_t n_groups;
    int32_t inner;       // groups per (sequence, tensor slot): position blocks x segments
    FastDiv inner_div;
    int32_t nseg;        // segments per row
    FastDiv seg_div;
    int32_t split;       // 1: one tensor per group, both present (tensor = (gid / inner) & 1)
    int32_t tens0;       // the tensor when one tensor per group and only one present
    int32_t xcd_per;     // workgroups per XCD (grid / 8) when renumbering by XCD, else 0
    FastDiv page_div;
};

__device__ __forceinline__ int32_t group_index(const GroupGeom& g) {
    const int32_t bid = (int32_t)blockIdx.x;
    const int32_t xb = (bid & 7) * g.xcd_per + (bid >> 3);
    return (g.xcd_per ? xb : bid) * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// group -> (sequence b, tensor of a one-tensor group, index within the
// (sequence, tensor) slot); no branch, so every kernel-argument load of the
// wave issues at once.  Padding groups (gid >= n_groups) take the last group
// and are reported dead.
__device__ __forceinline__ bool decode_group(const GroupGeom& g, int32_t& b, int32_t& tensor, int32_t& k) {
    const int32_t raw = group_index(g);
    const bool ok = raw < g.n_groups;
    const int32_t gid = ok ? raw : g.n_groups - 1;
    const int32_t rest = (int32_t)fast_div((uint32_t)gid, g.inner_div);
    k = gid - rest * g.inner;
    tensor = g.split ? (rest & 1) : g.tens0;
    b = rest >> g.split;
    return ok;
}

// ================================================================ fp16 -> compact, block per lane
//
// R % 1024 == 0.  A wave converts units NU k .. NU k + NU - 1 of one
// (sequence, tensor): unit u is position u / nseg, segment u % nseg (units
// past the last are dead).  Load instruction i fetches 16 bytes per lane:
// unit i >> 1, chunk (i & 1) * 64 + l of that unit.  The units are quantized
// in pairs; within pair q = i >> 2, chunk c = 64 (i & 3) + l goes to slot
// (c & 3) * 66 + (c >> 2) of the pair's LDS region, so lane L later reads
// its block's chunks 4L .. 4L + 3 from slots j * 66 + L (consecutive lanes,
// consecutive slots); the stride of 66 keeps the 8 lanes of each write
// phase in different banks.  Lanes 0..31 hold the blocks of the pair's
// first unit, lanes 32..63 those of its second.

constexpr int kLdsSlots = 3 * 66 + 64;   // 16-byte slots per wave

__device__ __forceinline__ uint32_t absmax_block(const uint4 (&v)[4]) {
    const uint32_t w[16] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                            v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
    return absmax_words(w);
}

// Codes of the block in v (32 elements, this lane), packed: Q4 in c[0..3],
// Q6 in c[0..5] (two 12-byte groups of 16 codes), Q8 in c[0..7]; returns
// the block's stored scale.
template <int WBITS>
__device__ __forceinline__ uint32_t quant_block(const uint4 (&v)[4], uint32_t (&c)[8]) {
    const uint32_t s16 = scale_from_absmax<WBITS>(absmax_block(v));
    const ScaleOps so = prep_scale(s16);
    uint32_t u[4][8];
    quant_chunks<WBITS, 4>(v, s16, so, u);
    if constexpr (WBITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = pack_q4(u[k]);
        c[4] = c[5] = c[6] = c[7] = 0;
    } else if constexpr (WBITS == 8) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c[2 * k] = pack_q8x4(u[k][0], u[k][1], u[k][2], u[k][3]);
            c[2 * k + 1] = pack_q8x4(u[k][4], u[k][5], u[k][6], u[k][7]);
        }
    } else {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pack_q6(u[k], lo[k], hi[k]);
        c[0] = lo[0];
        c[1] = __builtin_amdgcn_perm(lo[1], hi[0], 0x05040100u);   // hi0.lo16 | lo1.lo16 << 16
        c[2] = __builtin_amdgcn_alignbit(hi[1], lo[1], 16);        // lo1 >> 16 | hi1 << 16
        c[3] = lo[2];
        c[4] = __builtin_amdgcn_perm(lo[3], hi[2], 0x05040100u);
        c[5] = __builtin_amdgcn_alignbit(hi[3], lo[3], 16);
        c[6] = c[7] = 0;
    }
    return s16;
}

// FMT: 0 (8-bit high byte), 4, 6 or 8 -- the format of the group's tensor.
// The wave converts NU (2 or 4) consecutive units of one tensor, loaded
// together and quantized as NU / 2 pairs; wl is the wave's NU / 2 LDS
// regions (one per pair).
template <int FMT, int MODE, int NU>
__device__ __forceinline__ void narrow_run(const QLaunch& a, const GroupGeom& g, uint4 (*wl)[kLdsSlots],
                                           bool gok, int32_t b, int32_t tensor, int32_t k) {
    static_assert(NU == 2 || NU == 4, "two or four units per wave");
    const int lane = threadIdx.x & 63;
    const int32_t R = a.R;
    const int32_t units = a.width * g.nseg;
    int32_t t[NU], seg[NU], dt[NU];
    bool in[NU];
#pragma unroll
    for (int h = 0; h < NU; ++h) {
        const int32_t u = NU * k + h;   // unit NU * k is always in range (k < ceil(units / NU))
        in[h] = u < units;
        const int32_t uu = in[h] ? u : units - 1;
        t[h] = (int32_t)fast_div((uint32_t)uu, g.seg_div);
        seg[h] = uu - t[h] * g.nseg;
    }
#pragma unroll
    for (int h = 0; h < NU; ++h) dt[h] = t[h] - t[0];   // in [0, NU): consecutive units
    int64_t rr[NU], row[NU];
    bool live[NU];
    resolve_positions<MODE, NU>(a, g.page_div, b, t[0], dt, in, rr);
#pragma unroll
    for (int h = 0; h < NU; ++h) {
        live[h] = gok && rr[h] >= 0;
        row[h] = rr[h] >= 0 ? rr[h] : 0;   // skipped units read row 0 and store nothing
    }
    const uint16_t* src = static_cast<const uint16_t*>(tensor ? a.v_src : a.k_src);
    uint4 x[2 * NU];
#pragma unroll
    for (int i = 0; i < 2 * NU; ++i)
        x[i] = ld_nt(reinterpret_cast<const uint4*>(src + row[i >> 1] * R + seg[i >> 1] * 1024) + (i & 1) * 64 + lane);
    if constexpr (FMT == 0) {
        uint8_t* dst = static_cast<uint8_t*>(tensor ? a.v_dst : a.k_dst);
#pragma unroll
        for (int i = 0; i < 2 * NU; ++i) {
            const int h = i >> 1;
            const uint2 d = make_uint2(high_bytes(x[i].x, x[i].y), high_bytes(x[i].z, x[i].w));
            if (live[h]) st_nt(reinterpret_cast<uint2*>(dst + row[h] * R + seg[h] * 1024) + (i & 1) * 64 + lane, d);
        }
    } else {
        // pair q = i >> 2 holds units 2q, 2q + 1: its chunk c = 64 (i & 3) + l
#pragma unroll
        for (int i = 0; i < 2 * NU; ++i) {
            const int c = 64 * (i & 3) + lane;
            wl[i >> 2][(c & 3) * 66 + (c >> 2)] = x[i];
        }
        // the wave's own LDS writes are complete before it reads them back
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        const bool upper = lane >= 32;        // the lane's block lies in the pair's second unit
        uint8_t* codes = static_cast<uint8_t*>(tensor ? a.v_dst : a.k_dst);
        constexpr int32_t seg_code_bytes = 128 * FMT;     // a 1024-element segment's codes
#pragma unroll
        for (int q = 0; q < NU / 2; ++q) {
            const int h0 = 2 * q, h1 = 2 * q + 1;
            uint4 v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = wl[q][j * 66 + lane];
            const int64_t rowl = upper ? row[h1] : row[h0];
            const bool livel = upper ? live[h1] : live[h0];
            const int32_t blk = (upper ? seg[h1] : seg[h0]) * 32 + (lane & 31);
            uint32_t c[8];
            const uint32_t s16 = quant_block<FMT>(v, c);
            uint16_t* scales = static_cast<uint16_t*>(tensor ? a.v_scales : a.k_scales) + rowl * (int64_t)(R >> 5);
            if (livel) st_nt(scales + blk, s16);
            if constexpr (FMT == 4) {
                // 16 bytes per block: consecutive lanes, consecutive blocks
                if (livel)
                    st_nt(reinterpret_cast<uint4*>(codes + rowl * (int64_t)(R / 2)) + blk, make_uint4(c[0], c[1], c[2], c[3]));
            } else {
                // 24 or 32 bytes per block: stage the pair's codes (unit h0
                // then unit h1, each seg_code_bytes) in its LDS region and
                // store them as contiguous 16-byte lanes
                uint32_t* cw = reinterpret_cast<uint32_t*>(wl[q]);
                constexpr int W = FMT == 8 ? 8 : 6;           // dwords per block
#pragma unroll
                for (int i = 0; i < W; ++i) cw[lane * W + i] = c[i];
                __builtin_amdgcn_s_waitcnt(0xc07f);
                __builtin_amdgcn_wave_barrier();
                constexpr int pieces = 2 * seg_code_bytes / 16;   // 16-byte pieces of the pair's codes
#pragma unroll
                for (int i = 0; i < (pieces + 63) / 64; ++i) {
                    const int pc = 64 * i + lane;
                    if (pc < pieces) {
                        const uint4 d = wl[q][pc];
                        const bool second = pc * 16 >= seg_code_bytes;
                        const int32_t off = pc * 16 - (second ? seg_code_bytes : 0);
                        if (second ? live[h1] : live[h0])
                            st_nt(reinterpret_cast<uint4*>(codes + (second ? row[h1] : row[h0]) * (int64_t)(R / 8 * FMT) +
                                                           (int64_t)(second ? seg[h1] : seg[h0]) * seg_code_bytes + off),
                                  d);
                    }
                }
            }
        }
    }
}

// FMT >= 0: every present tensor has format FMT; -1: per-tensor formats,
// chosen per wave (a wave converts units of one tensor).
template <int FMT, int MODE, int NU>
__global__ __launch_bounds__(kThreads) void narrow_run_kernel(QLaunch a, GroupGeom g) {
    __shared__ uint4 lds[kWaves * (NU / 2)][kLdsSlots];
    int32_t b, tensor, k;
    const bool gok = decode_group(g, b, tensor, k);
    uint4 (*wl)[kLdsSlots] = lds + (threadIdx.x >> 6) * (NU / 2);
    if constexpr (FMT >= 0) {
        narrow_run<FMT, MODE, NU>(a, g, wl, gok, b, tensor, k);
    } else {
        switch (tensor ? a.fmt_v : a.fmt_k) {   // wave-uniform
            case 4: narrow_run<4, MODE, NU>(a, g, wl, gok, b, tensor, k); break;
            case 6: narrow_run<6, MODE, NU>(a, g, wl, gok, b, tensor, k); break;
            case 8: narrow_run<8, MODE, NU>(a, g, wl, gok, b, tensor, k); break;
            default: narrow_run<0, MODE, NU>(a, g, wl, gok, b, tensor, k); break;
        }
    }
}

// ================================================================ fp16 -> block codes, one unit per wave
//
// R % 1024 == 0, one common block format.  A wave converts one unit of one
// (sequence, tensor).  Its two loads are whole 1 KB runs (lane l: chunks l
// and 64 + l); an LDS pass hands lane l chunks 2l and 2l + 1 (16
// consecutive elements), so a 32-element block is a lane pair (its maximum
// one DPP exchange) and the lane's codes -- 8, 12 or 16 bytes -- are
// contiguous with its neighbours': every code store is a whole run, with no
// restaging.  Twice as many waves as the two-unit kernel, each with half the
// work.
template <int WBITS, int MODE>
__global__ __launch_bounds__(kThreads) void quant_lanepair_kernel(QLaunch a, GroupGeom g) {
    __shared__ uint4 lds[kWaves][128];
    uint4* wl = lds[threadIdx.x >> 6];
    int32_t b, tensor, k;
    const bool gok = decode_group(g, b, tensor, k);
    const int lane = threadIdx.x & 63;
    const int32_t R = a.R;
    const int32_t t = (int32_t)fast_div((uint32_t)k, g.seg_div);   // k < width * nseg: one unit per group
    const int32_t seg = k - t * g.nseg;
    const int32_t d[1] = {0};
    const bool tin[1] = {true};
    int64_t rr[1];
    resolve_positions<MODE, 1>(a, g.page_div, b, t, d, tin, rr);
    const bool live = gok && rr[0] >= 0;
    const int64_t row = rr[0] >= 0 ? rr[0] : 0;   // a skipped unit reads row 0 and stores nothing
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(tensor ? a.v_src : a.k_src) +
                                                      row * R + seg * 1024);
    const uint4 x0 = ld_nt(src + lane);
    const uint4 x1 = ld_nt(src + 64 + lane);
    wl[lane] = x0;
    wl[64 + lane] = x1;
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's own LDS writes are complete
    __builtin_amdgcn_wave_barrier();
    const uint4 v[2] = {wl[2 * lane], wl[2 * lane + 1]};
    const uint32_t s16 = scale_from_absmax<WBITS>(pair_max(absmax_2chunks(v[0], v[1])));
    const ScaleOps so = prep_scale(s16);
    uint32_t u[2][8];
    quant_chunks<WBITS, 2>(v, s16, so, u);
    uint8_t* c = static_cast<uint8_t*>(tensor ? a.v_dst : a.k_dst) + row * (int64_t)(R / 8 * WBITS) +
                 (int64_t)seg * (128 * WBITS);
    if constexpr (WBITS == 4) {
        if (live) st_nt(reinterpret_cast<uint2*>(c) + lane, make_uint2(pack_q4(u[0]), pack_q4(u[1])));
    } else if constexpr (WBITS == 8) {
        const uint4 q = make_uint4(pack_q8x4(u[0][0], u[0][1], u[0][2], u[0][3]), pack_q8x4(u[0][4], u[0][5], u[0][6], u[0][7]),
                                   pack_q8x4(u[1][0], u[1][1], u[1][2], u[1][3]), pack_q8x4(u[1][4], u[1][5], u[1][6], u[1][7]));
        if (live) st_nt(reinterpret_cast<uint4*>(c) + lane, q);
    } else {
        uint32_t lo0, hi0, lo1, hi1;
        pack_q6(u[0], lo0, hi0);
        pack_q6(u[1], lo1, hi1);
        const uint32_t d1 = __builtin_amdgcn_perm(lo1, hi0, 0x05040100u);   // hi0.lo16 | lo1.lo16 << 16
        const uint32_t d2 = __builtin_amdgcn_alignbit(hi1, lo1, 16);        // lo1 >> 16 | hi1 << 16
        if (live) st_nt3(c + 12 * lane, lo0, d1, d2);
    }
    uint16_t* scales = static_cast<uint16_t*>(tensor ? a.v_scales : a.k_scales);
    if (live && (lane & 1) == 0) st_nt(scales + row * (int64_t)(R >> 5) + seg * 32 + (lane >> 1), s16);
}

// ================================================================ compact -> fp16, runs of positions
//
// A group is (sequence b, block of P positions, segment) and NT tensors:
// both (NT = 2) or one (NT = 1).  Lane l holds chunks (8 elements)
// c = NCH * 64 * seg + 64 k + l, k < NCH, of each unit; GUARD masks the
// chunks past the row end of a partial last segment.

struct CodeChunk {
    uint32_t lo, hi;    // Q4: lo = 8 codes; Q6: the 8 bytes holding the 6 code bytes; Q8 / 8-bit: 8 codes
    uint32_t s;         // scale (fp16 bits)
};

// Q6, Q8 and 8-bit take unsigned 32-bit byte offsets from the wave-uniform
// row base (the scalar-base + vector-offset address form); Q4 keeps signed
// element offsets (full 64-bit addresses), measured faster for it: paged Q4
// 8.85 against 9.04 us, while the offset form gave Q6 10.30 against 10.76 us
// (with the branch-free shift below) and Q8 10.67 against 10.81 us.
template <int FMT, bool SCALE = true>
__device__ __forceinline__ CodeChunk load_code_chunk(const uint8_t* __restrict__ codes_row,
                                                     const uint16_t* __restrict__ scales_row, uint32_t c) {
    CodeChunk q;
    if constexpr (FMT == 4) {
        q.lo = ld_nt(reinterpret_cast<const uint32_t*>(codes_row) + (int32_t)c);
        q.hi = 0;
        q.s = SCALE ? ld_nt(scales_row + ((int32_t)c >> 2)) : 0u;
        return q;
    } else if constexpr (FMT == 8 || FMT == 0) {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(codes_row + 8u * c);
        q.lo = ld_nt(w);
        q.hi = ld_nt(w + 1);
    } else {
        // chunk c's 6 bytes start at 6c: load the 8 bytes of its 12-byte
        // group that contain them (4-byte aligned); odd chunks are shifted
        // into place after the load.
        const uint32_t* w = reinterpret_cast<const uint32_t*>(codes_row + (12u * (c >> 1) + 4u * (c & 1)));
        q.lo = ld_nt(w);
        q.hi = ld_nt(w + 1);
    }
    q.s = (FMT == 0 || !SCALE) ? 0u
                               : ld_nt(reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(scales_row) + 2u * (c >> 2)));
    return q;
}

// bytes 0,1 of w -> fp16 patterns byte << 8 in the low and high halves
__device__ __forceinline__ uint32_t widen_lo(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x01040004u); }
__device__ __forceinline__ uint32_t widen_hi(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x03040204u); }

template <int FMT>
__device__ __forceinline__ uint4 convert_chunk(const CodeChunk& q, uint32_t c) {
    if constexpr (FMT == 0) {
        return make_uint4(widen_lo(q.lo), widen_hi(q.lo), widen_lo(q.hi), widen_hi(q.hi));
    } else {
        const uint32_t s2 = q.s | (q.s << 16);
        if constexpr (FMT == 4) {
            return dequant_q4_chunk(q.lo, s2);
        } else if constexpr (FMT == 8) {
            return dequant_q8_chunk(q.lo, q.hi, s2);
        } else {
            // an odd chunk's 6 bytes start 2 bytes into the loaded 8: shift
            // by 16 bits, selected arithmetically (no divergent branch)
            const uint32_t sh = (c & 1u) << 4;
            const uint32_t lo = __builtin_amdgcn_alignbit(q.hi, q.lo, sh);
            const uint32_t hi = __builtin_amdgcn_ubfe(q.hi, sh, 16);
            return dequant_q6_chunk(lo, hi, s2);
        }
    }
}

__device__ __forceinline__ int64_t code_row_bytes(int fmt, int32_t R) { return fmt == 0 ? R : (int64_t)(R / 8) * fmt; }

template <int FMT, int MODE, int NCH, bool GUARD, int P, int NT>
__device__ __forceinline__ void widen_run(const QLaunch& a, const GroupGeom& g, uint2* __restrict__ wsc, bool gok,
                                          int32_t b, int32_t tsel, int32_t k) {
    const int32_t per_seq = MODE == kPrefix ? a.max_len : a.width;
    const int32_t tb = (int32_t)fast_div((uint32_t)k, g.seg_div);
    const int32_t seg = k - tb * g.nseg;
    int32_t d[P];
    bool tin[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        d[p] = p;
        tin[p] = tb * P + p < per_seq;
    }
    int64_t rr[P];
    resolve_positions<MODE, P>(a, g.page_div, b, tb * P, d, tin, rr);
    bool any = false;
#pragma unroll
    for (int p = 0; p < P; ++p) any = any || rr[p] >= 0;
    if (!(gok && any)) return;   // wave-uniform: grid padding, or every position skipped
    const int lane = threadIdx.x & 63;
    const int32_t R = a.R;
    const int32_t cpr = R >> 3;
    // Whole 1024-element segments: one 8-byte load per lane fetches every
    // scale of the wave's units (lane l: unit l / 8, scales 4 (l % 8) ..
    // + 3), staged through the wave's LDS slot, in place of one 2-byte load
    // per chunk.  Taken where it measured faster: runs of 8 Q6 / Q8 units
    // (paged Q6 9.66 against 10.21 us, Q8 10.25 against 10.60) and the full
    // prefix (128.6 against 131.5 us); Q4 runs lose 2% with it, one- and
    // two-unit paged waves up to 40%.
    constexpr int U = P * NT;
    constexpr bool STAGE = FMT > 0 && NCH == 2 && !GUARD && ((U == 8 && FMT != 4) || (MODE == kPrefix && U <= 8));
    if constexpr (STAGE) {
        const int uu = lane >> 3;
        const int up = uu / NT;
        int64_t urow = rr[0];
#pragma unroll
        for (int p = 1; p < P; ++p) urow = up == p ? rr[p] : urow;
        const int ut = NT == 2 ? (uu & 1) : tsel;
        const uint16_t* us = static_cast<const uint16_t*>(ut ? a.v_scales : a.k_scales) +
                             (urow >= 0 ? urow : 0) * (int64_t)(R >> 5) + seg * 32 + 4 * (lane & 7);
        if (uu < U) wsc[lane] = ld_nt(reinterpret_cast<const uint2*>(us));
    }
    CodeChunk q[P][NT][NCH];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int64_t row = rr[p] >= 0 ? rr[p] : 0;   // skipped positions read row 0 and store nothing
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int tensor = NT == 2 ? j : tsel;
            const uint8_t* codes = static_cast<const uint8_t*>(tensor ? a.v_src : a.k_src) + row * code_row_bytes(FMT, R);
            const uint16_t* scales =
                FMT == 0 ? nullptr : static_cast<const uint16_t*>(tensor ? a.v_scales : a.k_scales) + row * (int64_t)(R >> 5);
#pragma unroll
            for (int h = 0; h < NCH; ++h) {
                const uint32_t c = (uint32_t)(seg * (NCH * 64) + h * 64 + lane);
                if (GUARD) q[p][j][h] = c < (uint32_t)cpr ? load_code_chunk<FMT>(codes, scales, c) : CodeChunk{0, 0, 0};
                else q[p][j][h] = load_code_chunk<FMT, !STAGE>(codes, scales, c);
            }
        }
    }
    if constexpr (STAGE) {
        // the wave's own LDS writes are complete before it reads them back
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        const uint16_t* ws = reinterpret_cast<const uint16_t*>(wsc);
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int h = 0; h < NCH; ++h) q[p][j][h].s = ws[(p * NT + j) * 32 + h * 16 + (lane >> 2)];
    }
    // Stores go tensor by tensor: the P rows of one tensor are adjacent in
    // memory, so a wave writes one run per tensor rather than alternating
    // K and V rows (paged Q8 10.03 against 10.18 us, 8-bit 9.71 against
    // 10.07, per-layer Q4 8.68 against 8.97).
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tensor = NT == 2 ? j : tsel;
            uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(tensor ? a.v_dst : a.k_dst) +
                                                  (rr[p] >= 0 ? rr[p] : 0) * R);
#pragma unroll
            for (int h = 0; h < NCH; ++h) {
                const uint32_t c = (uint32_t)(seg * (NCH * 64) + h * 64 + lane);
                const uint4 o = convert_chunk<FMT>(q[p][j][h], c);
                if (rr[p] >= 0 && (!GUARD || c < (uint32_t)cpr)) st_nt(dst + c, o);
            }
        }
    }
}

// FMT >= 0: every present tensor has that format (0 = 8-bit); -1: per-tensor
// formats, one tensor per group (NT == 1).
template <int FMT, int MODE, int NCH, bool GUARD, int P, int NT>
__global__ __launch_bounds__(kThreads) void widen_run_kernel(QLaunch a, GroupGeom g) {
    __shared__ uint2 scale_lds[kWaves][64];   // per wave: the scales of up to 8 units
    uint2* wsc = scale_lds[threadIdx.x >> 6];
    int32_t b, tsel, k;
    const bool gok = decode_group(g, b, tsel, k);
    if constexpr (FMT >= 0) {
        widen_run<FMT, MODE, NCH, GUARD, P, NT>(a, g, wsc, gok, b, tsel, k);
    } else {
        static_assert(NT == 1, "per-tensor formats take one tensor per group");
        switch (tsel ? a.fmt_v : a.fmt_k) {   // wave-uniform
            case 4: widen_run<4, MODE, NCH, GUARD, P, 1>(a, g, wsc, gok, b, tsel, k); break;
            case 6: widen_run<6, MODE, NCH, GUARD, P, 1>(a, g, wsc, gok, b, tsel, k); break;
            case 8: widen_run<8, MODE, NCH, GUARD, P, 1>(a, g, wsc, gok, b, tsel, k); break;
            default: widen_run<0, MODE, NCH, GUARD, P, 1>(a, g, wsc, gok, b, tsel, k); break;
        }
    }
}

// ================================================================ contiguous 8-bit

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

// ================================================================ self-test kernels

// u[i * nx + j] = code of x[j] under scale s[i], through the same routines
// as the conversion kernels (one thread per chunk of 8 x values).
// CLAMP_ALL forces the clamping path; otherwise the kernels' dispatch on the
// scale is used.
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

// Plain non-temporal copy of n16 16-byte elements: a wave moves tiles of
// VPL x 64 consecutive elements (VPL loads per lane, all issued before its
// stores); waves stride over the tiles when the grid is smaller than the
// tile count.
template <int VPL, int WPB>
__global__ __launch_bounds__(64 * WPB) void selftest_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                                 int64_t n16) {
    const int64_t nw = (int64_t)gridDim.x * WPB;
    const int lane = threadIdx.x & 63;
    const int64_t tiles = (n16 + VPL * 64 - 1) / (VPL * 64);
    for (int64_t w = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6); w < tiles; w += nw) {
        const int64_t base = w * (VPL * 64) + lane;
        uint4 v[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t i = base + k * 64;
            v[k] = i < n16 ? ld_nt(src + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t i = base + k * 64;
            if (i < n16) st_nt(dst + i, v[k]);
        }
    }
}

// Uneven-traffic bandwidth references: per 64-lane tile each lane reads
// (GATHER) or writes (scatter) VPL 16-byte elements on the tile's heavy side
// and one element on its light side (the XOR of the elements read, or the
// element read written VPL times).  Heavy element k of lane l in tile w is
// w * 64 VPL + 64 k + l; its light element is w * 64 + l.
template <int VPL, int WPB, bool GATHER>
__global__ __launch_bounds__(64 * WPB) void selftest_stream_kernel(const uint4* __restrict__ src,
                                                                   uint4* __restrict__ dst, int64_t tiles) {
    const int64_t w = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    if (w >= tiles) return;
    const int lane = threadIdx.x & 63;
    const int64_t heavy = w * (VPL * 64) + lane;
    const int64_t light = w * 64 + lane;
    if constexpr (GATHER) {
        uint4 v[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) v[k] = ld_nt(src + heavy + 64 * k);
        uint4 acc = v[0];
#pragma unroll
        for (int k = 1; k < VPL; ++k) {
            acc.x ^= v[k].x;
            acc.y ^= v[k].y;
            acc.z ^= v[k].z;
            acc.w ^= v[k].w;
        }
        st_nt(dst + light, acc);
    } else {
        const uint4 x = ld_nt(src + light);
#pragma unroll
        for (int k = 0; k < VPL; ++k) st_nt(dst + heavy + 64 * k, x);
    }
}

// ================================================================ launchers

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

// The common format of the present tensors, or -1 when K and V differ.
static int common_format(const QLaunch& a) {
    const int fk = a.k_src ? a.fmt_k : -1, fv = a.v_src ? a.fmt_v : -1;
    if (fk < 0) return fv;
    return (fv < 0 || fv == fk) ? fk : -1;
}

// xcd: renumber workgroups by XCD (the grid is padded to a multiple of 8)
static int launch_groups(const void* fn, GroupGeom& g, bool xcd, QLaunch a, void* stream) {
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    int64_t grid = (g.n_groups + kWaves - 1) / kWaves;
    g.xcd_per = 0;
    if (xcd) {
        grid = (grid + 7) / 8 * 8;
        g.xcd_per = (int32_t)(grid / 8);
    }
    void* args[] = {&a, &g};
    return launch(fn, dim3((unsigned)grid), dim3(kThreads), args, stream);
}

// ---------------------------------------------------------------- fp16 -> compact

// Units per wave of the fp16 -> compact run kernel.  Four (two pairs, 8 KB
// of loads per wave) measured slower at every size tried, also with each
// pair converted while the next pair's loads were in flight: paged Q4 10.64
// against 9.53 us, paged 8-bit 11.31 against 10.63 us, contiguous 4 x 512
// positions 4.24 against 3.78 us.
constexpr int kNarrowUnits = 2;

template <int MODE>
static const void* narrow_run_fn(int fmt) {
    switch (fmt) {
        case 0: return reinterpret_cast<const void*>(&narrow_run_kernel<0, MODE, kNarrowUnits>);
        case 4: return reinterpret_cast<const void*>(&narrow_run_kernel<4, MODE, kNarrowUnits>);
        case 6: return reinterpret_cast<const void*>(&narrow_run_kernel<6, MODE, kNarrowUnits>);
        case 8: return reinterpret_cast<const void*>(&narrow_run_kernel<8, MODE, kNarrowUnits>);
        case -1: return reinterpret_cast<const void*>(&narrow_run_kernel<-1, MODE, kNarrowUnits>);
        default: return nullptr;
    }
}

// Renumber the run kernel's workgroups by XCD for paged launches (the waves
// of a sequence then share one L2 for its cache_seqlens and block_table
// lines).
static bool narrow_xcd(bool paged) { return paged; }

template <int MODE>
static const void* unit_fn(int fmt, bool guard) {
    if (fmt == 4) return guard ? reinterpret_cast<const void*>(&quant_unit_kernel<4, MODE, true>)
                               : reinterpret_cast<const void*>(&quant_unit_kernel<4, MODE, false>);
    if (fmt == 6) return guard ? reinterpret_cast<const void*>(&quant_unit_kernel<6, MODE, true>)
                               : reinterpret_cast<const void*>(&quant_unit_kernel<6, MODE, false>);
    if (fmt == 8) return guard ? reinterpret_cast<const void*>(&quant_unit_kernel<8, MODE, true>)
                               : reinterpret_cast<const void*>(&quant_unit_kernel<8, MODE, false>);
    return guard ? reinterpret_cast<const void*>(&narrow_unit_kernel<MODE, true>)
                 : reinterpret_cast<const void*>(&narrow_unit_kernel<MODE, false>);
}

template <int MODE>
static const void* lanepair_fn(int fmt) {
    switch (fmt) {
        case 4: return reinterpret_cast<const void*>(&quant_lanepair_kernel<4, MODE>);
        case 6: return reinterpret_cast<const void*>(&quant_lanepair_kernel<6, MODE>);
        case 8: return reinterpret_cast<const void*>(&quant_lanepair_kernel<8, MODE>);
        default: return nullptr;
    }
}

// One unit per wave (quant_lanepair_kernel) where it measured faster than
// two (narrow_run_kernel): every paged Q6 / Q8 launch, whose two-unit waves
// restage their codes through LDS (8 to 128 sequences x 256 positions: Q6
// 3.92 / 6.28 / 10.49 / 18.61 / 33.79 against 4.50 / 6.44 / 10.63 / 19.02 /
// 35.38 us, Q8 3.90 / 6.45 / 10.99 / 19.62 / 35.90 against 4.43 / 7.00 /
// 11.32 / 20.35 / 38.18 us), and any block format up to 4,096 units, where
// twice the waves fill more of the chip (paged Q4 at 8 x 256 positions 3.84
// against 4.20 us, contiguous 4 x 512 positions 3.23 against 3.35 us).
// Larger Q4 launches keep two units per wave (16 to 64 x 256 positions:
// 5.77 / 9.85 / 17.39 against 5.59 / 9.43 / 16.99 us), and so do larger
// contiguous ones (Q6 at 8 x 4,096 positions: 30.54 against 30.21 us).
static bool use_lanepair(int fmt, bool paged, int64_t units) {
    if (fmt != 4 && fmt != 6 && fmt != 8) return false;
    return units <= 4096 || (paged && fmt != 4);
}

static int launch_to_compact(const QLaunch& a, void* stream) {
    const bool paged = a.page_size != 0;
    const int fmt = common_format(a);
    const int ntens = (a.k_src ? 1 : 0) + (a.v_src ? 1 : 0);
    if (a.R % 1024 == 0 && use_lanepair(fmt, paged, (int64_t)a.batch * a.width * ntens * (a.R / 1024))) {
        GroupGeom g;
        g.nseg = a.R / 1024;
        g.seg_div = make_fastdiv((uint32_t)g.nseg);
        g.inner = (int32_t)((int64_t)a.width * g.nseg);   // one unit per group
        g.inner_div = make_fastdiv((uint32_t)g.inner);
        g.split = ntens == 2 ? 1 : 0;
        g.tens0 = a.k_src ? 0 : 1;
        g.n_groups = (int32_t)((int64_t)a.batch * ntens * g.inner);   // bounded by the host checks
        g.page_div = make_fastdiv(paged ? (uint32_t)a.page_size : 1u);
        const void* fn = paged ? lanepair_fn<kPaged>(fmt) : lanepair_fn<kContig>(fmt);
        return launch_groups(fn, g, narrow_xcd(paged), a, stream);
    }
    if (a.R % 1024 == 0) {
        // two units of one tensor per wave, also when K and V have
        // different formats (the wave takes its tensor's: K-Q4 + V-Q6 at
        // 64 x 256 positions 18.40 against 18.98 us one unit per wave)
        GroupGeom g;
        g.nseg = a.R / 1024;
        g.seg_div = make_fastdiv((uint32_t)g.nseg);
        const int64_t units = (int64_t)a.width * g.nseg;
        g.inner = (int32_t)((units + kNarrowUnits - 1) / kNarrowUnits);
        g.inner_div = make_fastdiv((uint32_t)g.inner);
        g.split = ntens == 2 ? 1 : 0;
        g.tens0 = a.k_src ? 0 : 1;
        g.n_groups = (int32_t)((int64_t)a.batch * ntens * g.inner);   // bounded by the host checks
        g.page_div = make_fastdiv(paged ? (uint32_t)a.page_size : 1u);
        const void* fn = paged ? narrow_run_fn<kPaged>(fmt) : narrow_run_fn<kContig>(fmt);
        // XCD renumbering: at the paged Q4 size 9.65 against 9.71 us, for
        // layer caches with a shared table 9.68 against 9.85 us, 128 x 256
        // positions 31.9 against 33.1 us; contiguous launches lose (3.94
        // against 3.88 us for 4 x 512 positions, 33.3 against 31.9 us for
        // 8 x 4096 positions of Q6)
        return launch_groups(fn, g, narrow_xcd(paged), a, stream);
    }
    // one unit per wave: the row's 16-element pieces, guarded when they are
    // not a multiple of 64
    const bool guard = (a.R / 16) % 64 != 0;
    QGeom g;
    g.nseg = (a.R + 1023) / 1024;
    g.ntens = ntens;
    g.tens0 = a.k_src ? 0 : 1;
    g.n_units = (int32_t)((int64_t)a.batch * a.width * g.ntens * g.nseg);   // bounded by the host checks
    g.seq_div = make_fastdiv((uint32_t)a.width);
    g.page_div = make_fastdiv(paged ? (uint32_t)a.page_size : 1u);
    const dim3 grid((unsigned)((g.n_units + kWaves - 1) / kWaves));
    QLaunch arg = a;
    void* args[] = {&arg, &g};
    const void* fn;
    if (fmt > 0) fn = paged ? unit_fn<kPaged>(fmt, guard) : unit_fn<kContig>(fmt, guard);
    else fn = paged ? unit_fn<kPaged>(-1, guard) : unit_fn<kContig>(-1, guard);   // per-tensor switch (or 8-bit)
    return launch(fn, grid, dim3(kThreads), args, stream);
}

// ---------------------------------------------------------------- compact -> fp16
//
// Paged launches of 8,192 to 32,768 units run P = 2, 4 or 8 positions
// with both tensors (about 2,048 waves), or P = 8 positions of one tensor,
// per wave: a single resident generation whose waves each keep several
// units in flight, so every lookup finishes before the chip's memory
// queues fill.
// Other paged launches take one position per wave: small ones to fill the
// chip, large ones because many short waves stream better over several
// generations (both tensors of a position in one wave, sharing the lookup).
// Full-prefix launches run 4 positions at 8,192 to 16,384 units.
// Contiguous K + V launches up to 16,384 units take 2 positions per wave up
// to 8,192 units and 8 above; larger ones one unit per wave.
// Measured at the paged Q4 size (16,384 units): 8.97 us for 4 positions x 2
// tensors per wave with XCD renumbering, against 10.67 us for one position;
// at 32,768 units 18.4 against 19.2 us, at 65,536 units 35.8 against 35.1;
// for the full-prefix widen of the same caches (~530,000 units): 135 us for
// one position x 2 tensors, 148 us for 4 positions, 158 us with XCD
// renumbering; contiguous Q6 at 65,536 units: 32.1 us for one unit per wave,
// 33.3 us for two.

template <int FMT, int MODE, int NCH, bool GUARD>
static const void* widen_fn(int P, int NT) {
    // the (P, NT) shapes the launcher picks; any other gets no kernel (the
    // launch then fails) rather than one whose grid would not match
    if (NT == 1 && P == 1) return reinterpret_cast<const void*>(&widen_run_kernel<FMT, MODE, NCH, GUARD, 1, 1>);
    if (NT == 1 && P == 8) return reinterpret_cast<const void*>(&widen_run_kernel<FMT, MODE, NCH, GUARD, 8, 1>);
    if (NT == 2 && P == 1) return reinterpret_cast<const void*>(&widen_run_kernel<FMT, MODE, NCH, GUARD, 1, 2>);
    if (NT == 2 && P == 4) return reinterpret_cast<const void*>(&widen_run_kernel<FMT, MODE, NCH, GUARD, 4, 2>);
    if constexpr (MODE != kPrefix) {
        if (NT == 2 && P == 2) return reinterpret_cast<const void*>(&widen_run_kernel<FMT, MODE, NCH, GUARD, 2, 2>);
        if (NT == 2 && P == 8) return reinterpret_cast<const void*>(&widen_run_kernel<FMT, MODE, NCH, GUARD, 8, 2>);
    }
    return nullptr;
}

template <int MODE, int NCH, bool GUARD>
static const void* widen_fn_fmt(int fmt, int P, int NT) {
    switch (fmt) {
        case 0: return widen_fn<0, MODE, NCH, GUARD>(P, NT);
        case 4: return widen_fn<4, MODE, NCH, GUARD>(P, NT);
        case 6: return widen_fn<6, MODE, NCH, GUARD>(P, NT);
        case 8: return widen_fn<8, MODE, NCH, GUARD>(P, NT);
        default:   // per-tensor formats: one tensor per group
            if (NT == 1 && P == 1) return reinterpret_cast<const void*>(&widen_run_kernel<-1, MODE, NCH, GUARD, 1, 1>);
            if (NT == 1 && P == 8) return reinterpret_cast<const void*>(&widen_run_kernel<-1, MODE, NCH, GUARD, 8, 1>);
            return nullptr;
    }
}

template <int MODE>
static const void* widen_fn_mode(int fmt, int nch, bool guard, int P, int NT) {
    if (guard) return widen_fn_fmt<MODE, 2, true>(fmt, P, NT);
    return nch == 2 ? widen_fn_fmt<MODE, 2, false>(fmt, P, NT) : widen_fn_fmt<MODE, 1, false>(fmt, P, NT);
}

static int launch_to_fp16(const QLaunch& a, int mode, void* stream) {
    const int fmt = common_format(a);
    const int ntens = (a.k_src ? 1 : 0) + (a.v_src ? 1 : 0);
    const int32_t cpr = a.R >> 3;
    int nch = 2;
    bool guard = false;
    if (cpr % 128 == 0) nch = 2;
    else if (cpr % 64 == 0) nch = 1;
    else guard = true;
    const int32_t per_seq = mode == kPrefix ? a.max_len : a.width;
    GroupGeom g;
    g.nseg = (cpr + nch * 64 - 1) / (nch * 64);
    g.seg_div = make_fastdiv((uint32_t)g.nseg);
    const int64_t units = (int64_t)a.batch * per_seq * ntens * g.nseg;
    // one tensor per group when the present tensors' formats differ, and for
    // large contiguous launches (no lookup to share, more waves to spread)
    const int NT = (fmt < 0 || ntens == 1 || (mode == kContig && units > 16384)) ? 1 : 2;
    // paged K + V runs up to 32,768 units still fit one resident generation
    // (one-tensor runs of 8 positions measured slower there: 20.9 against
    // 19.3 us for K-Q4 + V-Q6 at 64 x 256 positions)
    const bool run = units >= 8192 && units <= (mode == kPaged && NT == 2 ? 32768 : 16384);
    int P = run ? (NT == 2 ? 4 : 8) : 1;
    // paged K + V runs keep about 2,048 waves: 2 positions per wave below
    // 12,288 units (16 x 256 positions: Q4 5.06 against 5.30 us, Q8 5.74
    // against 6.02, 8-bit 5.41 against 5.74), 8 from 24,576 units for Q4
    // and 8-bit (64 x 256 positions: 17.39 against 18.26 us, 8-bit 19.46
    // against 20.10); Q6 and Q8 keep 4 there, where their 8-unit waves stage
    // the scales (Q6 with 8 positions 19.40 against 18.95 us)
    if (run && mode == kPaged && NT == 2) {
        if (units < 12288) P = 2;
        else if (units >= 24576 && (fmt == 4 || fmt == 0)) P = 8;
    }
    // contiguous K + V launches up to 16,384 units: 2 positions per wave up
    // to 8,192 units, 8 above (4 x 512 positions: 3.35 against 4.09 us for
    // one position; 4 x 2,048 positions: 8.01 against 8.53 us for 4)
    if (mode == kContig && NT == 2 && units <= 16384) P = units <= 8192 ? 2 : 8;
    const int64_t tblocks = (per_seq + P - 1) / P;
    g.inner = (int32_t)(tblocks * g.nseg);
    g.inner_div = make_fastdiv((uint32_t)g.inner);
    g.split = (NT == 1 && ntens == 2) ? 1 : 0;
    g.tens0 = a.k_src ? 0 : 1;
    g.n_groups = (int32_t)((int64_t)a.batch * (g.split ? 2 : 1) * g.inner);   // bounded by the host checks
    g.page_div = make_fastdiv(mode == kContig ? 1u : (uint32_t)a.page_size);
    const void* fn = mode == kPaged    ? widen_fn_mode<kPaged>(fmt, nch, guard, P, NT)
                     : mode == kPrefix ? widen_fn_mode<kPrefix>(fmt, nch, guard, P, NT)
                                       : widen_fn_mode<kContig>(fmt, nch, guard, P, NT);
    // renumbering by XCD pays off for every paged launch (128 x 256
    // positions, one position per wave: 34.4 against 35.1 us) and for
    // full-prefix runs, not for the one-position full-prefix launches
    // (155 against 131 us) whose dead waves it gathers
    return launch_groups(fn, g, mode == kPaged || (mode == kPrefix && run), a, stream);
}

int launch_quant_kv(const QLaunch& a, void* stream) { return launch_to_compact(a, stream); }

int launch_dequant_kv(const QLaunch& a, void* stream) {
    return launch_to_fp16(a, a.page_size ? kPaged : kContig, stream);
}

int launch_fp16_to_kv(const QLaunch& a, void* stream) { return launch_to_compact(a, stream); }

int launch_kv_to_fp16(const QLaunch& a, void* stream) {
    return launch_to_fp16(a, a.page_size ? kPaged : kContig, stream);
}

int launch_kv_to_fp16_prefix(const QLaunch& a, void* stream) { return launch_to_fp16(a, kPrefix, stream); }

// ---------------------------------------------------------------- self-tests

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

template <int VPL>
static const void* copy_fn(int wpb) {
    if (wpb == 1) return reinterpret_cast<const void*>(&selftest_copy_kernel<VPL, 1>);
    if (wpb == 2) return reinterpret_cast<const void*>(&selftest_copy_kernel<VPL, 2>);
    if (wpb == 4) return reinterpret_cast<const void*>(&selftest_copy_kernel<VPL, 4>);
    return reinterpret_cast<const void*>(&selftest_copy_kernel<VPL, 8>);
}

int launch_selftest_copy(const void* src, void* dst, int64_t n16, int lane_bytes, int group_waves, int64_t max_waves,
                         void* stream) {
    const int vpl = lane_bytes / 16;
    const int64_t tiles = (n16 + vpl * 64 - 1) / (vpl * 64);
    const int64_t waves = max_waves > 0 && max_waves < tiles ? max_waves : tiles;
    const dim3 grid((unsigned)((waves + group_waves - 1) / group_waves));
    void* args[] = {&src, &dst, &n16};
    const void* fn = vpl == 1 ? copy_fn<1>(group_waves) : vpl == 2 ? copy_fn<2>(group_waves)
                   : vpl == 4 ? copy_fn<4>(group_waves) : copy_fn<8>(group_waves);
    return launch(fn, grid, dim3(64 * group_waves), args, stream);
}

template <int VPL, bool GATHER>
static const void* stream_fn(int wpb) {
    if (wpb == 1) return reinterpret_cast<const void*>(&selftest_stream_kernel<VPL, 1, GATHER>);
    if (wpb == 2) return reinterpret_cast<const void*>(&selftest_stream_kernel<VPL, 2, GATHER>);
    if (wpb == 4) return reinterpret_cast<const void*>(&selftest_stream_kernel<VPL, 4, GATHER>);
    return reinterpret_cast<const void*>(&selftest_stream_kernel<VPL, 8, GATHER>);
}

template <bool GATHER>
static const void* stream_fn(int vpl, int wpb) {
    return vpl == 2 ? stream_fn<2, GATHER>(wpb) : vpl == 4 ? stream_fn<4, GATHER>(wpb) : stream_fn<8, GATHER>(wpb);
}

int launch_selftest_stream(const void* src, void* dst, int64_t tiles, int lane_elems, int group_waves, bool gather,
                           void* stream) {
    const dim3 grid((unsigned)((tiles + group_waves - 1) / group_waves));
    void* args[] = {&src, &dst, &tiles};
    const void* fn = gather ? stream_fn<true>(lane_elems, group_waves) : stream_fn<false>(lane_elems, group_waves);
    return launch(fn, grid, dim3(64 * group_waves), args, stream);
}

}  // namespace kvq
