// kvq_kernels.hip -- gfx950 kernels of the KV-cache format conversions and
// their launchers.
//
// Operations: ExLlamaV2 cache page, Description of fp16_to_fp8 /
// fp8_to_fp16 / fp16_to_q_kv / q_to_fp16_kv (contiguous windows and paged
// caches addressed through block_table / cache_seqlens).
//
// Work decomposition
//   8-bit: each span (one sequence's window) is a contiguous run of
//     width * R elements; threads stream 8-element chunks with 128-bit
//     fp16 accesses and 64-bit byte accesses.
//   Q4/Q6: one wavefront per token row (row segment of up to 1024 elements)
//     handles that row of K and of V; lane l holds chunks l and l + 64, so a
//     32-element block is one DPP quad and a 1024-element row needs no loop.
//     The physical row is resolved once per wave from scalar loads of
//     cache_seqlens / block_table.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kWaves = 4;                 // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kNch = 2;                   // chunks per lane per row segment
constexpr int kSegChunks = 64 * kNch;     // 1024 elements per wave
constexpr int kFp8Cpt = 4;                // chunks per thread, 8-bit kernels

// ---------------------------------------------------------------- row map

// Physical row of logical row n = b * width + t, or -1 when skipped.
// Contiguous: (b, offset + t).  Paged: position p = cache_seqlens[b] +
// offset + t in page block_table[b][p / page_size], slot p % page_size;
// skipped if p < 0, past the table, or the page is outside [0, dim0).
// All values are wave-uniform (scalar loads and SALU).
__device__ __forceinline__ int64_t resolve_row(const QLaunch& a, int32_t n) {
    const int32_t b = n / a.width;
    const int32_t t = n - b * a.width;
    if (a.page_size == 0) return (int64_t)b * a.dim1 + a.offset + t;
    const int64_t p = (int64_t)a.cache_seqlens[b] + a.offset + t;
    if (p < 0 || p >= (int64_t)a.bt_cols * a.page_size) return -1;
    const uint32_t pu = (uint32_t)p;
    const uint32_t pi = pu / (uint32_t)a.page_size;
    const int32_t page = a.block_table[(int64_t)b * a.bt_cols + pi];
    if (page < 0 || page >= a.dim0) return -1;
    return (int64_t)page * a.page_size + (int64_t)(pu - pi * (uint32_t)a.page_size);
}

// Scale operands for the element routine.  A zero scale maps every element
// to q = 0: with (s, r) = (1, 0), y = 0, e = x and y2 = 0.
__device__ __forceinline__ void prep_scale(uint32_t s16, float& s, float& r) {
    const float sf = h2f(s16);
    const bool zero = (sf == 0.0f);
    s = zero ? 1.0f : sf;
    r = zero ? 0.0f : __builtin_amdgcn_rcpf(sf);
}

// ---------------------------------------------------------------- quantize

template <int WBITS>
__device__ __forceinline__ void quant_store_chunk(uint4 x, int32_t c, bool active, int lane,
                                                  uint8_t* __restrict__ codes_row,
                                                  uint16_t* __restrict__ scales_row) {
    const uint32_t s16 = scale_from_absmax<WBITS>(quad_max(absmax_chunk(x)));
    float s, r;
    prep_scale(s16, s, r);
    uint32_t u[8];
    quant_chunk<WBITS>(x, s16, s, r, u);
    if constexpr (WBITS == 4) {
        const uint32_t w = pack_q4(u);
        if (active) reinterpret_cast<uint32_t*>(codes_row)[c] = w;
    } else {
        uint32_t lo, hi;
        pack_q6(u, lo, hi);
        // lanes 2m, 2m+1 own one 12-byte group: the even lane writes bytes
        // 0..7, the odd lane bytes 8..11.
        const uint32_t partner_lo = pair_swap(lo);
        if (active) {
            if ((lane & 1) == 0) {
                uint2 d;
                d.x = lo;
                d.y = __builtin_amdgcn_perm(partner_lo, hi, 0x05040100u);   // hi.lo16 | partner.lo16 << 16
                __builtin_memcpy(codes_row + 6 * c, &d, 8);   // 4-byte aligned
            } else {
                const uint32_t d = __builtin_amdgcn_alignbit(hi, lo, 16);   // lo >> 16 | hi << 16
                *reinterpret_cast<uint32_t*>(codes_row + 6 * c + 2) = d;
            }
        }
    }
    if (active && (lane & 3) == 0) scales_row[c >> 2] = (uint16_t)s16;
}

template <int WBITS>
__global__ __launch_bounds__(kThreads) void quant_kv_kernel(QLaunch a, int32_t nseg,
                                                            int32_t n_units) {
    const int lane = threadIdx.x & 63;
    const int32_t unit = (int32_t)blockIdx.x * kWaves +
                         __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (unit >= n_units) return;
    int32_t n = unit, g = 0;
    if (nseg > 1) {
        n = unit / nseg;
        g = unit - n * nseg;
    }
    const int64_t row = resolve_row(a, n);
    if (row < 0) return;

    const int32_t R = a.R;
    const int32_t cpr = R >> 3;
    const int32_t cbase = g * kSegChunks + lane;
    const int64_t elem0 = row * R;
    const int64_t code0 = row * (int64_t)(R / 8 * WBITS);
    const int64_t scale0 = row * (int64_t)(R >> 5);

    const uint4* ksrc = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_src) + elem0);
    const uint4* vsrc = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_src) + elem0);
    const bool has_k = a.k_src != nullptr;
    const bool has_v = a.v_src != nullptr;

    uint4 kx[kNch], vx[kNch];
#pragma unroll
    for (int k = 0; k < kNch; ++k) {
        const int32_t c = cbase + k * 64;
        kx[k] = make_uint4(0, 0, 0, 0);
        vx[k] = make_uint4(0, 0, 0, 0);
        if (c < cpr) {
            if (has_k) kx[k] = ksrc[c];
            if (has_v) vx[k] = vsrc[c];
        }
    }
    if (has_k) {
        uint8_t* codes = static_cast<uint8_t*>(a.k_dst) + code0;
        uint16_t* scales = static_cast<uint16_t*>(a.k_scales) + scale0;
#pragma unroll
        for (int k = 0; k < kNch; ++k) {
            const int32_t c = cbase + k * 64;
            quant_store_chunk<WBITS>(kx[k], c, c < cpr, lane, codes, scales);
        }
    }
    if (has_v) {
        uint8_t* codes = static_cast<uint8_t*>(a.v_dst) + code0;
        uint16_t* scales = static_cast<uint16_t*>(a.v_scales) + scale0;
#pragma unroll
        for (int k = 0; k < kNch; ++k) {
            const int32_t c = cbase + k * 64;
            quant_store_chunk<WBITS>(vx[k], c, c < cpr, lane, codes, scales);
        }
    }
}

// ---------------------------------------------------------------- dequantize

struct CodeChunk {
    uint32_t lo, hi;    // Q4: lo = 8 codes; Q6: 48-bit field (lo, hi16)
    uint32_t s2;        // scale replicated in both halves
};

template <int WBITS>
__device__ __forceinline__ CodeChunk load_code_chunk(const uint8_t* __restrict__ codes_row,
                                                     const uint16_t* __restrict__ scales_row,
                                                     int32_t c) {
    CodeChunk q;
    if constexpr (WBITS == 4) {
        q.lo = reinterpret_cast<const uint32_t*>(codes_row)[c];
        q.hi = 0;
    } else {
        // chunk c's 6 bytes start at 6c; load the 8 bytes of its 12-byte
        // group that contain them (4-byte aligned) and shift odd chunks.
        uint2 d;
        __builtin_memcpy(&d, codes_row + 12 * (c >> 1) + 4 * (c & 1), 8);
        if (c & 1) {
            q.lo = __builtin_amdgcn_alignbit(d.y, d.x, 16);
            q.hi = d.y >> 16;
        } else {
            q.lo = d.x;
            q.hi = d.y & 0xFFFFu;
        }
    }
    const uint32_t s = scales_row[c >> 2];
    q.s2 = s | (s << 16);
    return q;
}

template <int WBITS>
__device__ __forceinline__ uint4 dequant_chunk(const CodeChunk& q) {
    if constexpr (WBITS == 4) return dequant_q4_chunk(q.lo, q.s2);
    else return dequant_q6_chunk(q.lo, q.hi, q.s2);
}

template <int WBITS>
__global__ __launch_bounds__(kThreads) void dequant_kv_kernel(QLaunch a, int32_t nseg,
                                                              int32_t n_units) {
    const int lane = threadIdx.x & 63;
    const int32_t unit = (int32_t)blockIdx.x * kWaves +
                         __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (unit >= n_units) return;
    int32_t n = unit, g = 0;
    if (nseg > 1) {
        n = unit / nseg;
        g = unit - n * nseg;
    }
    const int64_t row = resolve_row(a, n);
    if (row < 0) return;

    const int32_t R = a.R;
    const int32_t cpr = R >> 3;
    const int32_t cbase = g * kSegChunks + lane;
    const int64_t elem0 = row * R;
    const int64_t code0 = row * (int64_t)(R / 8 * WBITS);
    const int64_t scale0 = row * (int64_t)(R >> 5);
    const bool has_k = a.k_src != nullptr;
    const bool has_v = a.v_src != nullptr;

    CodeChunk kq[kNch], vq[kNch];
#pragma unroll
    for (int k = 0; k < kNch; ++k) {
        const int32_t c = cbase + k * 64;
        kq[k] = CodeChunk{0, 0, 0};
        vq[k] = CodeChunk{0, 0, 0};
        if (c < cpr) {
            if (has_k)
                kq[k] = load_code_chunk<WBITS>(static_cast<const uint8_t*>(a.k_src) + code0,
                                               static_cast<const uint16_t*>(a.k_scales) + scale0, c);
            if (has_v)
                vq[k] = load_code_chunk<WBITS>(static_cast<const uint8_t*>(a.v_src) + code0,
                                               static_cast<const uint16_t*>(a.v_scales) + scale0, c);
        }
    }
#pragma unroll
    for (int k = 0; k < kNch; ++k) {
        const int32_t c = cbase + k * 64;
        if (c < cpr) {
            if (has_k)
                reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.k_dst) + elem0)[c] =
                    dequant_chunk<WBITS>(kq[k]);
            if (has_v)
                reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.v_dst) + elem0)[c] =
                    dequant_chunk<WBITS>(vq[k]);
        }
    }
}

// ---------------------------------------------------------------- 8-bit

// high byte of each fp16: bytes 1,3 of the first word then 1,3 of the second
__device__ __forceinline__ uint32_t high_bytes(uint32_t w0, uint32_t w1) {
    return __builtin_amdgcn_perm(w1, w0, 0x07050301u);
}

// bytes 0,1 of w -> fp16 patterns byte << 8 in the low and high halves
__device__ __forceinline__ uint32_t widen_lo(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x01040004u); }
__device__ __forceinline__ uint32_t widen_hi(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x03040204u); }

__global__ __launch_bounds__(kThreads) void fp16_to_fp8_kernel(Fp8Launch a) {
    const int64_t cps = a.span_elems >> 3;
    const int64_t c0 = (int64_t)blockIdx.x * (kThreads * kFp8Cpt) + threadIdx.x;
    for (int32_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const int64_t e0 = (int64_t)b * a.batch_stride_elems + a.first_elem;
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.in) + e0);
        uint2* dst = reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.out) + e0);
        uint4 v[kFp8Cpt];
#pragma unroll
        for (int k = 0; k < kFp8Cpt; ++k) {
            const int64_t c = c0 + k * kThreads;
            v[k] = c < cps ? src[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kFp8Cpt; ++k) {
            const int64_t c = c0 + k * kThreads;
            if (c < cps) dst[c] = make_uint2(high_bytes(v[k].x, v[k].y), high_bytes(v[k].z, v[k].w));
        }
    }
}

__global__ __launch_bounds__(kThreads) void fp8_to_fp16_kernel(Fp8Launch a) {
    const int64_t cps = a.span_elems >> 3;
    const int64_t c0 = (int64_t)blockIdx.x * (kThreads * kFp8Cpt) + threadIdx.x;
    for (int32_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const int64_t e0 = (int64_t)b * a.batch_stride_elems + a.first_elem;
        const uint2* src = reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a.in) + e0);
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + e0);
        uint2 v[kFp8Cpt];
#pragma unroll
        for (int k = 0; k < kFp8Cpt; ++k) {
            const int64_t c = c0 + k * kThreads;
            v[k] = c < cps ? src[c] : make_uint2(0, 0);
        }
#pragma unroll
        for (int k = 0; k < kFp8Cpt; ++k) {
            const int64_t c = c0 + k * kThreads;
            if (c < cps)
                dst[c] = make_uint4(widen_lo(v[k].x), widen_hi(v[k].x), widen_lo(v[k].y), widen_hi(v[k].y));
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
    float s, r;
    prep_scale(s16[i], s, r);
    uint32_t c[8];
    if (CLAMP_ALL) quant_chunk_impl<WBITS, true>(v, s, r, c);
    else quant_chunk<WBITS>(v, s16[i], s, r, c);
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

// ---------------------------------------------------------------- launchers

static int launch(const void* fn, dim3 grid, dim3 block, void** args, void* stream) {
    return (int)hipLaunchKernel(fn, grid, block, args, 0, static_cast<hipStream_t>(stream));
}

static dim3 fp8_grid(const Fp8Launch& a) {
    const int64_t cps = a.span_elems >> 3;
    const int64_t gx = (cps + kThreads * kFp8Cpt - 1) / (kThreads * kFp8Cpt);
    const int32_t gy = a.batch < 65535 ? a.batch : 65535;
    return dim3((unsigned)gx, (unsigned)gy, 1);
}

int launch_fp16_to_fp8(const Fp8Launch& a, void* stream) {
    Fp8Launch arg = a;
    void* args[] = {&arg};
    return launch(reinterpret_cast<const void*>(&fp16_to_fp8_kernel), fp8_grid(a), dim3(kThreads), args, stream);
}

int launch_fp8_to_fp16(const Fp8Launch& a, void* stream) {
    Fp8Launch arg = a;
    void* args[] = {&arg};
    return launch(reinterpret_cast<const void*>(&fp8_to_fp16_kernel), fp8_grid(a), dim3(kThreads), args, stream);
}

static void q_geometry(const QLaunch& a, int32_t& nseg, int32_t& n_units, dim3& grid) {
    const int32_t cpr = a.R >> 3;
    nseg = (cpr + kSegChunks - 1) / kSegChunks;
    n_units = (int32_t)((int64_t)a.batch * a.width * nseg);   // bounded by the host checks
    grid = dim3((unsigned)((n_units + kWaves - 1) / kWaves), 1, 1);
}

int launch_quant_kv(const QLaunch& a, void* stream) {
    QLaunch arg = a;
    int32_t nseg, n_units;
    dim3 grid;
    q_geometry(a, nseg, n_units, grid);
    void* args[] = {&arg, &nseg, &n_units};
    const void* fn = a.wbits == 4 ? reinterpret_cast<const void*>(&quant_kv_kernel<4>)
                                  : reinterpret_cast<const void*>(&quant_kv_kernel<6>);
    return launch(fn, grid, dim3(kThreads), args, stream);
}

int launch_dequant_kv(const QLaunch& a, void* stream) {
    QLaunch arg = a;
    int32_t nseg, n_units;
    dim3 grid;
    q_geometry(a, nseg, n_units, grid);
    void* args[] = {&arg, &nseg, &n_units};
    const void* fn = a.wbits == 4 ? reinterpret_cast<const void*>(&dequant_kv_kernel<4>)
                                  : reinterpret_cast<const void*>(&dequant_kv_kernel<6>);
    return launch(fn, grid, dim3(kThreads), args, stream);
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
    else
        fn = force_clamp ? reinterpret_cast<const void*>(&selftest_codes_kernel<6, true>)
                         : reinterpret_cast<const void*>(&selftest_codes_kernel<6, false>);
    return launch(fn, grid, dim3(kThreads), args, stream);
}

int launch_selftest_scales(const uint16_t* a, int64_t n, int wbits, uint16_t* out, void* stream) {
    dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    void* args[] = {&a, &n, &out};
    const void* fn = wbits == 4 ? reinterpret_cast<const void*>(&selftest_scales_kernel<4>)
                                : reinterpret_cast<const void*>(&selftest_scales_kernel<6>);
    return launch(fn, grid, dim3(kThreads), args, stream);
}

}  // namespace kvq
