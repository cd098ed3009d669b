// kvq_internal.h -- launch descriptors shared by the host API and the HIP
// launchers.  Plain C++ (no HIP types), so the validation layer stays
// host-only code.
#pragma once

#include <stdint.h>

namespace kvq {

// One call of the fp16 <-> 8-bit conversion: `batch` spans of `span_elems`
// contiguous elements; span b starts at element b * batch_stride_elems.
struct Fp8Launch {
    const void* in;
    void* out;
    int64_t batch_stride_elems;   // dim1 * R
    int64_t first_elem;           // offset * R
    int64_t span_elems;           // width * R (a multiple of 8)
    int32_t batch;
};

// One call of the K/V block (de)quantization.  For quantization `k_src` /
// `v_src` are fp16 caches and `k_dst` / `v_dst` code buffers; for
// dequantization the roles swap.  Scales are written by quantization and read
// by dequantization.  A NULL source skips that half.
struct QLaunch {
    const void* k_src; void* k_dst; void* k_scales;
    const void* v_src; void* v_dst; void* v_scales;
    int32_t dim0, dim1;           // physical shape (pages x page_size when paged)
    int32_t R;                    // elements per token row (heads * head_dim, % 32 == 0)
    int32_t batch, offset, width;
    int32_t page_size;            // 0: contiguous
    const int32_t* cache_seqlens; // paged only
    const int32_t* block_table;   // paged only, [batch, bt_cols]
    int32_t bt_cols;
    int32_t wbits;                // single-width calls
    int32_t fmt_k, fmt_v;         // per-tensor calls: 0 = 8-bit high byte, 4/6/8 = block codes
    int32_t max_len;              // full-prefix calls: positions enumerated per sequence
};

// Division by a run-time constant d (1 <= d < 2^31) without a divide, for
// numerators 0 <= n < 2^31 (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994, Theorem 4.2, with N = 32):
//   l = ceil(log2 d),  m = floor(2^(32+l) / d) + 1 = 2^32 + mul,
//   floor(n / d) = floor(m n / 2^(32+l)) = (mulhi(n, mul) + n) >> l.
// The theorem needs 2^(32+l) <= m d <= 2^(32+l) + 2^l, which holds because
// 2^(32+l) < m d <= 2^(32+l) + d and d <= 2^l; mulhi(n, mul) < n keeps the
// sum below 2^32 for n < 2^31.
struct FastDiv {
    uint32_t mul;
    uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while (l < 31 && (1u << l) < d) ++l;
    FastDiv f;
    f.mul = (uint32_t)((((uint64_t)1 << l) - d) * ((uint64_t)1 << 32) / d + 1);
    f.shift = l;
    return f;
}

// Launchers (return a hipError_t value as int, 0 on success).
int launch_fp16_to_fp8(const Fp8Launch& a, void* stream);
int launch_fp8_to_fp16(const Fp8Launch& a, void* stream);
int launch_quant_kv(const QLaunch& a, void* stream);
int launch_dequant_kv(const QLaunch& a, void* stream);
int launch_fp16_to_kv(const QLaunch& a, void* stream);
int launch_kv_to_fp16(const QLaunch& a, void* stream);
int launch_kv_to_fp16_prefix(const QLaunch& a, void* stream);

// Element-level self-test launchers (same device routines as the kernels).
int launch_selftest_codes(const uint16_t* x, int64_t nx, const uint16_t* s, int64_t ns,
                          int wbits, bool force_clamp, uint8_t* u, void* stream);
int launch_selftest_scales(const uint16_t* a, int64_t n, int wbits, uint16_t* out, void* stream);
int launch_selftest_fastdiv(const uint32_t* n, int64_t count, uint32_t d, uint32_t* q, void* stream);
// Plain non-temporal copy of n16 16-byte elements (bandwidth reference).
int launch_selftest_copy(const void* src, void* dst, int64_t n16, int lane_bytes, int group_waves, int64_t max_waves,
                         void* stream);
// Uneven-traffic reference: `tiles` tiles of 64 lanes, lane_elems 16-byte
// elements per lane on the heavy side (read when gathering, written when
// scattering), one on the light side.
int launch_selftest_stream(const void* src, void* dst, int64_t tiles, int lane_elems, int group_waves, bool gather,
                           void* stream);

}  // namespace kvq
