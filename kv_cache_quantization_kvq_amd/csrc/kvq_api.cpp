// kvq_api.cpp -- the C ABI declared in include/kvq.h: argument validation,
// dispatch to the HIP launchers, and the host-side count_match.
//
// Operations and arguments: ExLlamaV2 cache page, Signature and I/O Contract
// (batch_size, offset, width, page_size, cache_seqlens, block_table, wbits;
// dtype checks kHalf <-> kUInt8).  Validation happens entirely on the host,
// before anything is enqueued.
//
// (The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
// Exllamav2 Ext Cache".)
#include <stdint.h>
#include <string.h>

#include <climits>

#include "../../include/kvq.h"
#include "../../include/kvq_selftest.h"
#include "kvq_internal.h"

namespace {

using kvq::Fp8Launch;
using kvq::QLaunch;

constexpr int64_t kMaxRowElems = 1 << 20;
// A launch's work-items per grid dimension (workgroups x threads) must fit
// the 32-bit grid size of the dispatch packet; the bounds below keep every
// launch under it with room for the last partial workgroup and, for the K/V
// calls, for padding the grid to a multiple of 8 workgroups.
constexpr int64_t kMaxWorkItems = (INT64_C(1) << 32) - 1024;
constexpr int64_t kMaxUnits = ((INT64_C(1) << 32) - 4096) / 64;   // at most one 64-lane wavefront per unit
constexpr int64_t kMaxCacheElems = INT64_C(1) << 60;    // dim0 * dim1 * heads * head_dim
// Positions a block-table row addresses (block_table_cols * page_size): the
// kernels test positions in 32-bit arithmetic with this headroom.
constexpr int64_t kMaxPositions = INT64_C(1) << 30;

// a * b for a, b >= 0, saturated at INT64_MAX (extents of the overlap check)
int64_t sat_mul(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Extent {
    const void* p;
    int64_t bytes;
    bool is_output;
};

bool overlaps(const Extent& x, const Extent& y) {
    if (!x.p || !y.p || x.bytes <= 0 || y.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), a1 = a0 + (uintptr_t)x.bytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(y.p), b1 = b0 + (uintptr_t)y.bytes;
    return a0 < b1 && b0 < a1;
}

// Any output extent overlapping any other extent of the call.
bool any_output_overlap(const Extent* e, int n) {
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if ((e[i].is_output || e[j].is_output) && overlaps(e[i], e[j])) return true;
    return false;
}

// Common shape/window checks.  q_path: head_dim % 32 == 0 (block formats
// and the per-tensor calls); otherwise the row length % 8 == 0 (contiguous
// 8-bit path).
int check_shape(const kvq_shape& s, bool q_path) {
    if (s.dim0 <= 0 || s.dim1 <= 0 || s.heads <= 0 || s.head_dim <= 0) return KVQ_ERR_SHAPE;
    const int64_t R = (int64_t)s.heads * s.head_dim;
    if (R > kMaxRowElems) return KVQ_ERR_SHAPE;
    if (q_path ? (s.head_dim % 32 != 0) : (R % 8 != 0)) return KVQ_ERR_SHAPE;
    if ((int64_t)s.dim0 * s.dim1 > kMaxCacheElems / R) return KVQ_ERR_RANGE;
    return KVQ_OK;
}

int check_contig_window(const kvq_shape& s, int batch_size, int offset, int width) {
    if (batch_size < 0 || offset < 0 || width < 0) return KVQ_ERR_RANGE;
    if (batch_size > s.dim0) return KVQ_ERR_RANGE;
    if ((int64_t)offset + width > s.dim1) return KVQ_ERR_RANGE;
    return KVQ_OK;
}

int fp8_call(bool to_fp8, const void* in, void* out, kvq_shape s, int batch_size, int offset,
             int width, void* stream) {
    if (!in || !out) return KVQ_ERR_NULL;
    int rc = check_shape(s, false);
    if (rc) return rc;
    rc = check_contig_window(s, batch_size, offset, width);
    if (rc) return rc;
    if (!aligned(in, 16) || !aligned(out, 16)) return KVQ_ERR_ALIGN;
    const int64_t R = (int64_t)s.heads * s.head_dim;
    const int64_t elems = (int64_t)s.dim0 * s.dim1 * R;
    const Extent ext[2] = {{in, elems * (to_fp8 ? 2 : 1), false}, {out, elems * (to_fp8 ? 1 : 2), true}};
    if (any_output_overlap(ext, 2)) return KVQ_ERR_OVERLAP;
    if ((int64_t)width * R / 8 > kMaxWorkItems) return KVQ_ERR_RANGE;   // one thread per 8 elements at most
    if (batch_size == 0 || width == 0) return KVQ_OK;
    Fp8Launch a;
    a.in = in;
    a.out = out;
    a.batch_stride_elems = (int64_t)s.dim1 * R;
    a.first_elem = (int64_t)offset * R;
    a.span_elems = (int64_t)width * R;
    a.batch = batch_size;
    const int err = to_fp8 ? kvq::launch_fp16_to_fp8(a, stream) : kvq::launch_fp8_to_fp16(a, stream);
    return err ? KVQ_ERR_HIP : KVQ_OK;
}

bool valid_fmt(int f) { return f == 0 || f == 4 || f == 6 || f == 8; }

// bytes of one row's compact form and of its scales, for format f
int64_t compact_row_bytes(int64_t R, int f) { return f == 0 ? R : R / 8 * f; }
int64_t scale_row_bytes(int64_t R, int f) { return f == 0 ? 0 : (R / 32) * 2; }

enum CallKind { kSingleWidth, kPerTensor, kPrefixWiden };

// Shared validation and dispatch of every K/V conversion.  to_compact: fp16
// sources, compact destinations; otherwise the reverse.  For kSingleWidth
// fmt_k == fmt_v == wbits; for kPrefixWiden offset is unused and max_len
// bounds the positions per sequence.
int kv_call(CallKind kind, bool to_compact, const void* k_src, void* k_dst, const void* k_scales, int fmt_k,
            const void* v_src, void* v_dst, const void* v_scales, int fmt_v, kvq_shape s, int batch_size,
            int offset, int width, int page_size, int max_len, const int32_t* cache_seqlens,
            const int32_t* block_table, int block_table_cols, void* stream) {
    const bool k_present = k_src || k_dst, v_present = v_src || v_dst;
    if (kind == kSingleWidth) {
        const bool k_any = k_present || k_scales, v_any = v_present || v_scales;
        if ((k_any && !(k_src && k_dst && k_scales)) || (v_any && !(v_src && v_dst && v_scales)) ||
            (!k_any && !v_any))
            return KVQ_ERR_NULL;
    } else {
        if ((k_present && !(k_src && k_dst)) || (v_present && !(v_src && v_dst)) || (!k_present && !v_present))
            return KVQ_ERR_NULL;
        if ((k_present && !valid_fmt(fmt_k)) || (v_present && !valid_fmt(fmt_v))) return KVQ_ERR_WBITS;
        if (k_present && ((fmt_k == 0) != (k_scales == nullptr))) return KVQ_ERR_NULL;
        if (v_present && ((fmt_v == 0) != (v_scales == nullptr))) return KVQ_ERR_NULL;
        if (!k_present && k_scales) return KVQ_ERR_NULL;
        if (!v_present && v_scales) return KVQ_ERR_NULL;
    }
    int rc = check_shape(s, true);
    if (rc) return rc;
    if (kind == kPrefixWiden) {
        page_size = s.dim1;
        if (batch_size < 0 || width < 0 || max_len < 0 || block_table_cols <= 0) return KVQ_ERR_RANGE;
    } else if (page_size < 0) {
        return KVQ_ERR_RANGE;
    }
    if (page_size == 0) {
        rc = check_contig_window(s, batch_size, offset, width);
        if (rc) return rc;
    } else {
        if (page_size != s.dim1) return KVQ_ERR_SHAPE;
        if (batch_size < 0 || offset < 0 || width < 0 || block_table_cols <= 0) return KVQ_ERR_RANGE;
        if ((int64_t)block_table_cols * page_size > kMaxPositions) return KVQ_ERR_RANGE;
        if (!cache_seqlens || !block_table) return KVQ_ERR_NULL;
        if (!aligned(cache_seqlens, 4) || !aligned(block_table, 4)) return KVQ_ERR_ALIGN;
    }
    const int64_t R = (int64_t)s.heads * s.head_dim;
    // work units (row segments of K and V), one wavefront each
    const int64_t max_seg = (R / 8 + 63) / 64;
    const int64_t per_seq = kind == kPrefixWiden ? max_len : width;
    if ((int64_t)batch_size * per_seq > kMaxUnits || (int64_t)batch_size * per_seq * 2 * max_seg > kMaxUnits)
        return KVQ_ERR_RANGE;
    const void* ptrs[6] = {k_src, k_dst, k_scales, v_src, v_dst, v_scales};
    for (const void* p : ptrs)
        if (p && !aligned(p, 16)) return KVQ_ERR_ALIGN;

    const int64_t rows = (int64_t)s.dim0 * s.dim1;
    auto f16b = [&](void) { return rows * R * 2; };
    const int64_t k_compact = rows * compact_row_bytes(R, fmt_k), v_compact = rows * compact_row_bytes(R, fmt_v);
    const Extent ext[8] = {
        {k_src, to_compact ? f16b() : k_compact, false}, {k_dst, to_compact ? k_compact : f16b(), true},
        {k_scales, rows * scale_row_bytes(R, fmt_k), to_compact},
        {v_src, to_compact ? f16b() : v_compact, false}, {v_dst, to_compact ? v_compact : f16b(), true},
        {v_scales, rows * scale_row_bytes(R, fmt_v), to_compact},
        {cache_seqlens, page_size ? (int64_t)batch_size * 4 : 0, false},
        {block_table, page_size ? sat_mul((int64_t)batch_size * block_table_cols, 4) : 0, false}};
    if (any_output_overlap(ext, 8)) return KVQ_ERR_OVERLAP;
    if (batch_size == 0 || per_seq == 0) return KVQ_OK;

    QLaunch a;
    a.k_src = k_present ? k_src : nullptr; a.k_dst = k_present ? k_dst : nullptr;
    a.k_scales = const_cast<void*>(k_scales);
    a.v_src = v_present ? v_src : nullptr; a.v_dst = v_present ? v_dst : nullptr;
    a.v_scales = const_cast<void*>(v_scales);
    a.dim0 = s.dim0; a.dim1 = s.dim1; a.R = (int32_t)R;
    a.batch = batch_size; a.offset = kind == kPrefixWiden ? 0 : offset; a.width = width;
    a.page_size = page_size;
    a.cache_seqlens = page_size ? cache_seqlens : nullptr;
    a.block_table = page_size ? block_table : nullptr;
    a.bt_cols = page_size ? block_table_cols : 0;
    a.wbits = fmt_k;
    a.fmt_k = fmt_k; a.fmt_v = fmt_v;
    a.max_len = max_len;
    int err;
    if (kind == kSingleWidth) err = to_compact ? kvq::launch_quant_kv(a, stream) : kvq::launch_dequant_kv(a, stream);
    else if (kind == kPerTensor) err = to_compact ? kvq::launch_fp16_to_kv(a, stream) : kvq::launch_kv_to_fp16(a, stream);
    else err = kvq::launch_kv_to_fp16_prefix(a, stream);
    return err ? KVQ_ERR_HIP : KVQ_OK;
}

int q_call(bool quant, const void* k_src, void* k_dst, const void* k_scales, const void* v_src,
           void* v_dst, const void* v_scales, kvq_shape s, int batch_size, int offset, int width,
           int page_size, const int32_t* cache_seqlens, const int32_t* block_table,
           int block_table_cols, int wbits, void* stream) {
    if (wbits != 4 && wbits != 6 && wbits != 8) return KVQ_ERR_WBITS;
    return kv_call(kSingleWidth, quant, k_src, k_dst, k_scales, wbits, v_src, v_dst, v_scales, wbits, s,
                   batch_size, offset, width, page_size, 0, cache_seqlens, block_table, block_table_cols,
                   stream);
}

}  // namespace

extern "C" {

int kvq_fp16_to_fp8(const void* in_f16, void* out_u8, kvq_shape s, int batch_size, int offset,
                    int width, void* hip_stream) {
    return fp8_call(true, in_f16, out_u8, s, batch_size, offset, width, hip_stream);
}

int kvq_fp8_to_fp16(const void* in_u8, void* out_f16, kvq_shape s, int batch_size, int offset,
                    int width, void* hip_stream) {
    return fp8_call(false, in_u8, out_f16, s, batch_size, offset, width, hip_stream);
}

int kvq_fp16_to_q_kv(const void* k_in, void* k_out, void* k_scales, const void* v_in, void* v_out,
                     void* v_scales, kvq_shape s, int batch_size, int offset, int width,
                     int page_size, const int32_t* cache_seqlens, const int32_t* block_table,
                     int block_table_cols, int wbits, void* hip_stream) {
    return q_call(true, k_in, k_out, k_scales, v_in, v_out, v_scales, s, batch_size, offset, width,
                  page_size, cache_seqlens, block_table, block_table_cols, wbits, hip_stream);
}

int kvq_q_to_fp16_kv(const void* k_in, void* k_out, const void* k_scales, const void* v_in,
                     void* v_out, const void* v_scales, kvq_shape s, int batch_size, int offset,
                     int width, int page_size, const int32_t* cache_seqlens,
                     const int32_t* block_table, int block_table_cols, int wbits,
                     void* hip_stream) {
    return q_call(false, k_in, k_out, k_scales, v_in, v_out, v_scales, s, batch_size, offset, width,
                  page_size, cache_seqlens, block_table, block_table_cols, wbits, hip_stream);
}

int kvq_fp16_to_kv(const void* k_in, void* k_out, void* k_scales, int fmt_k, const void* v_in,
                   void* v_out, void* v_scales, int fmt_v, kvq_shape s, int batch_size, int offset,
                   int width, int page_size, const int32_t* cache_seqlens, const int32_t* block_table,
                   int block_table_cols, void* hip_stream) {
    return kv_call(kPerTensor, true, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, s,
                   batch_size, offset, width, page_size, 0, cache_seqlens, block_table, block_table_cols,
                   hip_stream);
}

int kvq_kv_to_fp16(const void* k_in, void* k_out, const void* k_scales, int fmt_k, const void* v_in,
                   void* v_out, const void* v_scales, int fmt_v, kvq_shape s, int batch_size, int offset,
                   int width, int page_size, const int32_t* cache_seqlens, const int32_t* block_table,
                   int block_table_cols, void* hip_stream) {
    return kv_call(kPerTensor, false, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, s,
                   batch_size, offset, width, page_size, 0, cache_seqlens, block_table, block_table_cols,
                   hip_stream);
}

int kvq_kv_to_fp16_prefix(const void* k_in, void* k_out, const void* k_scales, int fmt_k,
                          const void* v_in, void* v_out, const void* v_scales, int fmt_v, kvq_shape s,
                          int batch_size, int width, int max_len, const int32_t* cache_seqlens,
                          const int32_t* block_table, int block_table_cols, void* hip_stream) {
    return kv_call(kPrefixWiden, false, k_in, k_out, k_scales, fmt_k, v_in, v_out, v_scales, fmt_v, s,
                   batch_size, 0, width, s.dim1, max_len, cache_seqlens, block_table, block_table_cols,
                   hip_stream);
}

int64_t kvq_bytes_per_token(int format, int heads, int head_dim) {
    if (format != 16 && !valid_fmt(format)) return KVQ_ERR_WBITS;
    if (heads <= 0 || head_dim <= 0) return KVQ_ERR_SHAPE;
    if (format != 16 && format != 0 && head_dim % 32 != 0) return KVQ_ERR_SHAPE;
    const int64_t R = (int64_t)heads * head_dim;
    if (format == 16) return 2 * R;
    return compact_row_bytes(R, format) + scale_row_bytes(R, format);
}

// Matching prefix in 64-bit chunks (ExLlamaV2 cache page, Description of
// count_match): whole 8-byte words are compared four at a time, the first
// differing word is then resolved element by element.
int64_t kvq_count_match(const void* a, int64_t len_a, const void* b, int64_t len_b, int64_t max_a,
                        int elem_bytes) {
    if (elem_bytes != 4 && elem_bytes != 8) return KVQ_ERR_RANGE;
    if (len_a < 0 || len_b < 0) return KVQ_ERR_RANGE;
    int64_t n = max_a < len_a ? max_a : len_a;
    if (len_b < n) n = len_b;
    if (n <= 0) return 0;
    if (!a || !b) return KVQ_ERR_NULL;
    const unsigned char* pa = static_cast<const unsigned char*>(a);
    const unsigned char* pb = static_cast<const unsigned char*>(b);
    const int64_t nbytes = n * elem_bytes;
    const int64_t nwords = nbytes / 8;
    int64_t w = 0;
    for (; w + 4 <= nwords; w += 4) {
        uint64_t x[4], y[4];
        memcpy(x, pa + 8 * w, 32);
        memcpy(y, pb + 8 * w, 32);
        if (((x[0] ^ y[0]) | (x[1] ^ y[1]) | (x[2] ^ y[2]) | (x[3] ^ y[3])) != 0) break;
    }
    for (; w < nwords; ++w) {
        uint64_t x, y;
        memcpy(&x, pa + 8 * w, 8);
        memcpy(&y, pb + 8 * w, 8);
        if (x != y) break;
    }
    // first element not covered by equal words
    int64_t i = (8 * w) / elem_bytes;
    for (; i < n; ++i)
        if (memcmp(pa + i * elem_bytes, pb + i * elem_bytes, (size_t)elem_bytes) != 0) return i;
    return n;
}

const char* kvq_strerror(int code) {
    switch (code) {
        case KVQ_OK: return "success";
        case KVQ_ERR_NULL: return "required pointer is NULL or a K/V triple is partial";
        case KVQ_ERR_WBITS: return "wbits must be 4, 6 or 8 (a format: KVQ_FMT_FP8, _Q4, _Q6 or _Q8)";
        case KVQ_ERR_SHAPE: return "invalid cache shape (head_dim % 32 for Q paths, heads*head_dim % 8 for 8-bit, page_size == dim1 when paged)";
        case KVQ_ERR_RANGE: return "size, offset or window out of range";
        case KVQ_ERR_ALIGN: return "device pointer not 16-byte aligned (int32 tables: 4)";
        case KVQ_ERR_OVERLAP: return "an output buffer overlaps another buffer of the call";
        case KVQ_ERR_HIP: return "HIP launch failed";
        default: return "unknown error";
    }
}

int kvq_version(void) { return 100; }

int kvq_selftest_codes(const uint16_t* x, int64_t nx, const uint16_t* s16, int64_t ns, int wbits,
                       int force_clamp, uint8_t* u_out, void* hip_stream) {
    if (wbits != 4 && wbits != 6 && wbits != 8) return KVQ_ERR_WBITS;
    if (!x || !s16 || !u_out) return KVQ_ERR_NULL;
    if (nx < 0 || ns < 0 || nx % 8 != 0) return KVQ_ERR_RANGE;
    if (!aligned(x, 16) || !aligned(u_out, 16) || !aligned(s16, 2)) return KVQ_ERR_ALIGN;
    if (nx == 0 || ns == 0) return KVQ_OK;
    if (nx / 8 > kMaxWorkItems / ns) return KVQ_ERR_RANGE;     // one thread per 8 x and scale
    return kvq::launch_selftest_codes(x, nx, s16, ns, wbits, force_clamp != 0, u_out, hip_stream)
               ? KVQ_ERR_HIP : KVQ_OK;
}

int kvq_selftest_scales(const uint16_t* absmax, int64_t n, int wbits, uint16_t* out, void* hip_stream) {
    if (wbits != 4 && wbits != 6 && wbits != 8) return KVQ_ERR_WBITS;
    if (!absmax || !out) return KVQ_ERR_NULL;
    if (n < 0 || n > kMaxWorkItems) return KVQ_ERR_RANGE;
    if (!aligned(absmax, 2) || !aligned(out, 2)) return KVQ_ERR_ALIGN;
    if (n == 0) return KVQ_OK;
    return kvq::launch_selftest_scales(absmax, n, wbits, out, hip_stream) ? KVQ_ERR_HIP : KVQ_OK;
}

int kvq_selftest_fastdiv(const uint32_t* n, int64_t count, uint32_t d, uint32_t* q, void* hip_stream) {
    if (!n || !q) return KVQ_ERR_NULL;
    if (d == 0 || d > (uint32_t)INT32_MAX || count < 0 || count > kMaxWorkItems) return KVQ_ERR_RANGE;
    if (!aligned(n, 4) || !aligned(q, 4)) return KVQ_ERR_ALIGN;
    if (count == 0) return KVQ_OK;
    return kvq::launch_selftest_fastdiv(n, count, d, q, hip_stream) ? KVQ_ERR_HIP : KVQ_OK;
}

int kvq_selftest_copy(const void* src, void* dst, int64_t bytes, int lane_bytes, int group_waves,
                      int64_t max_waves, void* hip_stream) {
    if (!src || !dst) return KVQ_ERR_NULL;
    if (bytes < 0 || bytes % 16 != 0 || max_waves < 0) return KVQ_ERR_RANGE;
    if (lane_bytes != 16 && lane_bytes != 32 && lane_bytes != 64 && lane_bytes != 128) return KVQ_ERR_RANGE;
    if (group_waves != 1 && group_waves != 2 && group_waves != 4 && group_waves != 8) return KVQ_ERR_RANGE;
    if (!aligned(src, 16) || !aligned(dst, 16)) return KVQ_ERR_ALIGN;
    const Extent ext[2] = {{src, bytes, false}, {dst, bytes, true}};
    if (any_output_overlap(ext, 2)) return KVQ_ERR_OVERLAP;
    if (bytes / 16 > kMaxWorkItems) return KVQ_ERR_RANGE;      // at most one 16-byte element per work-item
    if (bytes == 0) return KVQ_OK;
    return kvq::launch_selftest_copy(src, dst, bytes / 16, lane_bytes, group_waves, max_waves, hip_stream)
               ? KVQ_ERR_HIP : KVQ_OK;
}

int kvq_selftest_stream(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes, int lane_elems,
                        int group_waves, void* hip_stream) {
    if (!src || !dst) return KVQ_ERR_NULL;
    if (lane_elems != 2 && lane_elems != 4 && lane_elems != 8) return KVQ_ERR_RANGE;
    if (group_waves != 1 && group_waves != 2 && group_waves != 4 && group_waves != 8) return KVQ_ERR_RANGE;
    // sizes below 2^56, so the products below cannot overflow
    if (src_bytes < 0 || dst_bytes < 0 || src_bytes >= (INT64_C(1) << 56) || dst_bytes >= (INT64_C(1) << 56))
        return KVQ_ERR_RANGE;
    const bool gather = src_bytes == dst_bytes * lane_elems;
    const bool scatter = dst_bytes == src_bytes * lane_elems;
    if (!gather && !scatter) return KVQ_ERR_RANGE;
    const int64_t light = gather ? dst_bytes : src_bytes;
    if (light % 1024 != 0) return KVQ_ERR_RANGE;                 // whole 64-lane tiles of 16 bytes
    if (!aligned(src, 16) || !aligned(dst, 16)) return KVQ_ERR_ALIGN;
    const Extent ext[2] = {{src, src_bytes, false}, {dst, dst_bytes, true}};
    if (any_output_overlap(ext, 2)) return KVQ_ERR_OVERLAP;
    if (light / 16 > kMaxWorkItems) return KVQ_ERR_RANGE;       // one work-item per light-side element
    if (light == 0) return KVQ_OK;
    return kvq::launch_selftest_stream(src, dst, light / 1024, lane_elems, group_waves, gather, hip_stream)
               ? KVQ_ERR_HIP : KVQ_OK;
}

}  // extern "C"
