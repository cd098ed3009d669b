/*
 * kvq.h -- C ABI of the MI355X (gfx950) KV-cache format-conversion library.
 *
 * The operations are the five functions of the ExLlamaV2 cache extension as
 * described on the page "Implementation: Turboderp org Exllamav2 Ext Cache"
 * (sections Description, Signature, I/O Contract, Usage Examples):
 * fp16 <-> 8-bit, fp16 -> 4/6-bit block quantization of K and V with
 * per-block fp16 scales, its inverse, over contiguous or paged caches, and a
 * host-side matching-prefix count.  Tensors become raw pointers plus one
 * shape descriptor; the page's implicit "current stream" becomes an explicit
 * HIP stream argument.  Beyond the page's five functions: 8-bit block codes
 * (wbits 8), a format per tensor (paged 8-bit; K and V at different widths
 * in one launch), the widen of every cached position before attention, and
 * the bytes per token of each format.
 *
 * Conventions shared by every device call
 *   - All device pointers belong to the current HIP device and are owned by
 *     the caller.  The library allocates nothing, keeps no state between
 *     calls and writes outputs in place, touching only the rows the call
 *     covers; every other byte of an output buffer is left as it was.
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *     the default stream).  A kernel fault surfaces at the caller's next
 *     synchronisation with that stream.
 *   - The library launches through the HIP runtime it is linked against
 *     (libamdhip64.so.7).  Buffers and streams must come from the same runtime
 *     instance: a program that also uses another copy of the runtime (torch
 *     ships its own) must load that copy before this library, so that the
 *     dynamic loader binds both to it.
 *   - A call enqueues exactly one kernel launch (none when it has nothing to
 *     do) and no memory set, copy, allocation or synchronisation, so it may
 *     be captured into a HIP graph; replays reread the tables' current
 *     contents.  Calls that overlap in time (other streams, graph branches)
 *     are safe when they write disjoint rows or identical bytes.
 *   - Every base pointer of a device buffer must be 16-byte aligned
 *     (allocations from hipMalloc or torch satisfy this); int32 tables need
 *     4-byte alignment.
 *   - Return 0 on success or a negative KVQ_ERR_* code; nothing is printed
 *     and no exception crosses the ABI.  Arguments are validated on the host
 *     before any launch; on error nothing is enqueued.
 *   - batch_size == 0 or width == 0 validates the arguments and returns 0
 *     without launching.
 *   - Size limits: a row holds at most 2^20 elements (heads * head_dim), a
 *     cache at most 2^60 (dim0 * dim1 * heads * head_dim), a K/V call
 *     satisfies batch_size * width (max_len for the full prefix) * 2 *
 *     ceil(heads * head_dim / 512) <= 2^26 - 64, an 8-bit call converts at
 *     most (2^32 - 1024) * 8 elements per sequence window, and a paged table
 *     spans block_table_cols * page_size <= 2^30 positions.  (A K/V call runs
 *     at most one 64-lane wavefront per row segment of 512 or 1024 elements,
 *     a launch's work-items must fit the 32-bit grid size of a dispatch, and
 *     the kernels test positions in 32-bit arithmetic.)
 *
 * Layouts (row = one token: heads * head_dim elements, R below)
 *   fp16 cache     [dim0, dim1, heads, head_dim]            uint16 (fp16 bits)
 *   8-bit cache    [dim0, dim1, heads, head_dim]            uint8
 *   codes          [dim0, dim1, heads, head_dim * wbits/8]  uint8
 *   scales         [dim0, dim1, heads, head_dim / 32]       fp16
 *   Contiguous mode: dim0 = batch capacity, dim1 = sequence capacity.
 *   Paged mode:      dim0 = number of physical pages, dim1 = page_size.
 *
 * Numerics (the page fixes the operations, not the arithmetic; the
 * readings below are the library's definition):
 *   8-bit  byte = high byte of the fp16 pattern (e5m2, truncated toward 0);
 *          back: fp16 pattern = byte << 8.
 *   Q4/Q6/Q8  blocks of 32 consecutive elements along head_dim;
 *          s16 = fp16_rne(fp32(absmax) / (2^(b-1) - 1));
 *          q = 0 if s16 == 0, else clamp(round_half_even(x / s16),
 *              -2^(b-1), 2^(b-1) - 1); stored u = q + 2^(b-1);
 *          the codes of a row form one little-endian bit stream, code j at
 *          bits [b*j, b*j + b)  (4-bit: 8 codes per uint32 word; 6-bit: 16
 *          codes per 12 bytes; 8-bit: one code per byte).
 *   dequant x' = fp16_rne((float)(u - 2^(b-1)) * (float)s16).
 *   Inputs to the quantizer must be finite; scales given to the dequantizer
 *   must be finite.  Results are bit-identical across calls and devices.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points (the library is built with hidden visibility). */
#if defined(__GNUC__) || defined(__clang__)
#define KVQ_API __attribute__((visibility("default")))
#else
#define KVQ_API
#endif

#define KVQ_OK            0
#define KVQ_ERR_NULL     -1  /* a required pointer is NULL, or a K/V triple is partial */
#define KVQ_ERR_WBITS    -2  /* wbits not 4, 6 or 8 (or an unknown KVQ_FMT_* format) */
#define KVQ_ERR_SHAPE    -3  /* heads/head_dim/dims not positive, head_dim % 32 (Q) or
                                heads*head_dim % 8 (8-bit) not 0, paged page_size != dim1,
                                heads*head_dim > 2^20 */
#define KVQ_ERR_RANGE    -4  /* negative size or offset, window past dim0/dim1,
                                block_table_cols <= 0 in paged mode, elem_bytes not 4/8,
                                a size limit above exceeded */
#define KVQ_ERR_ALIGN    -5  /* a device base pointer is not 16-byte aligned (int32 tables: 4) */
#define KVQ_ERR_OVERLAP  -6  /* an output buffer overlaps another buffer of the call */
#define KVQ_ERR_HIP      -7  /* the HIP runtime rejected the launch */

/* Physical cache shape shared by all tensors of one call. */
typedef struct kvq_shape {
    int32_t dim0;       /* batch capacity (contiguous) or number of pages (paged) */
    int32_t dim1;       /* sequence capacity (contiguous) or page_size (paged) */
    int32_t heads;
    int32_t head_dim;
} kvq_shape;

/*
 * fp16 -> 8-bit over the contiguous window: rows (b, offset + t) for
 * b < batch_size, t < width.  ExLlamaV2 cache page, Description of
 * fp16_to_fp8 (fp16 cache tensors to the 8-bit format, unsigned bytes, strided 4D
 * layout with batch_size, offset, width for partial updates).
 *   in_f16  device, fp16 [dim0, dim1, heads, head_dim], read
 *   out_u8  device, uint8 of the same shape, written on the window only
 * Requires heads * head_dim % 8 == 0, batch_size <= dim0,
 * offset + width <= dim1.
 */
KVQ_API int kvq_fp16_to_fp8(const void* in_f16, void* out_u8, kvq_shape s,
                    int batch_size, int offset, int width, void* hip_stream);

/*
 * 8-bit -> fp16, the inverse of kvq_fp16_to_fp8 over the same window.
 * ExLlamaV2 cache page, Description of fp8_to_fp16 (validated and laid out
 * like the forward conversion).
 *   in_u8    device, uint8 [dim0, dim1, heads, head_dim], read
 *   out_f16  device, fp16 of the same shape, written on the window only
 */
KVQ_API int kvq_fp8_to_fp16(const void* in_u8, void* out_f16, kvq_shape s,
                    int batch_size, int offset, int width, void* hip_stream);

/*
 * fp16 -> 4/6/8-bit codes and per-block fp16 scales for K and V in one
 * launch.  ExLlamaV2 cache page, Description of fp16_to_q_kv (paged mode when
 * page_size > 0, using block_table and cache_seqlens; contiguous otherwise)
 * and I/O Contract (k_scales / v_scales: per-block scale factors; wbits 4 or
 * 6).  wbits 8 is the same block format with one code per byte, the width of
 * the page's ExLlamaV2Cache_Q8 class (Usage section).
 *   k_in, v_in          device, fp16 [dim0, dim1, heads, head_dim], read
 *   k_out, v_out        device, uint8 codes [dim0, dim1, heads, head_dim*wbits/8]
 *   k_scales, v_scales  device, fp16 [dim0, dim1, heads, head_dim/32], written
 *   Either triple may be all NULL to skip that half (at least one present);
 *   a partially NULL triple is KVQ_ERR_NULL.
 *   page_size == 0 (contiguous): rows (b, offset + t), b < batch_size <= dim0,
 *     t < width, offset + width <= dim1; cache_seqlens/block_table ignored.
 *   page_size  > 0 (paged, page_size == dim1): sequence b's position
 *     p = cache_seqlens[b] + offset + t lives in physical page
 *     block_table[b * block_table_cols + p / page_size], slot p % page_size.
 *     A row is skipped (not read, not written) when p < 0, when
 *     p / page_size >= block_table_cols, or when the page is outside
 *     [0, dim0).  cache_seqlens: device int32[batch_size]; block_table:
 *     device int32[batch_size, block_table_cols].  Two (b, t) mapping to the
 *     same physical row give an unspecified result.
 */
KVQ_API int kvq_fp16_to_q_kv(const void* k_in, void* k_out, void* k_scales,
                     const void* v_in, void* v_out, void* v_scales,
                     kvq_shape s, int batch_size, int offset, int width,
                     int page_size, const int32_t* cache_seqlens,
                     const int32_t* block_table, int block_table_cols,
                     int wbits, void* hip_stream);

/*
 * 4/6/8-bit codes + fp16 scales -> fp16 for K and V in one launch, over the
 * same rows as kvq_fp16_to_q_kv with the same arguments.  ExLlamaV2 cache
 * page, Description of q_to_fp16_kv (same paged/contiguous dual path) and
 * I/O Contract (k_out / v_out receive the fp16 values).
 *   k_in, v_in          device, uint8 codes [dim0, dim1, heads, head_dim*wbits/8], read
 *   k_out, v_out        device, fp16 [dim0, dim1, heads, head_dim], written
 *   k_scales, v_scales  device, fp16 [dim0, dim1, heads, head_dim/32], read
 */
KVQ_API int kvq_q_to_fp16_kv(const void* k_in, void* k_out, const void* k_scales,
                     const void* v_in, void* v_out, const void* v_scales,
                     kvq_shape s, int batch_size, int offset, int width,
                     int page_size, const int32_t* cache_seqlens,
                     const int32_t* block_table, int block_table_cols,
                     int wbits, void* hip_stream);

/*
 * Length of the matching prefix of two host arrays of elem_bytes-byte
 * elements (4 or 8), at most min(max_a, len_a, len_b) (0 when that is
 * negative).  ExLlamaV2 cache page, Description of count_match (CPU-side,
 * compares in 64-bit chunks, returns the matching prefix length, used for
 * prefix reuse in dynamic batching).  Counts elements of the given size.
 * Synchronous, host memory, no alignment requirement.  Returns the count, or
 * KVQ_ERR_NULL / KVQ_ERR_RANGE (negative lengths, elem_bytes not 4 or 8).
 */
KVQ_API int64_t kvq_count_match(const void* a, int64_t len_a, const void* b, int64_t len_b,
                        int64_t max_a, int elem_bytes);

/* ------------------------------------------------------------------------
 * Per-tensor formats.  The page's K/V functions take one wbits for both
 * tensors and its 8-bit functions have no paging arguments; the entry points
 * below take a format per tensor, so K and V may differ (one launch) and the
 * 8-bit format can be paged.  A tensor is present when its input and output
 * pointers are non-NULL (both, or neither); its scales pointer must be
 * non-NULL for the block formats and NULL for KVQ_FMT_FP8.  Shapes, rows,
 * paging and skipping are those of kvq_fp16_to_q_kv; head_dim % 32 == 0.
 * A format outside {FP8, Q4, Q6, Q8} is KVQ_ERR_WBITS.
 *   FP8 tensor: [dim0, dim1, heads, head_dim] uint8, no scales.
 *   Qb tensor:  codes [dim0, dim1, heads, head_dim*b/8] uint8 + fp16 scales
 *               [dim0, dim1, heads, head_dim/32].
 * ------------------------------------------------------------------------ */
#define KVQ_FMT_FP8    0   /* 8-bit: high byte of the fp16 pattern */
#define KVQ_FMT_Q4     4   /* 4-bit block codes + fp16 scale per 32 elements */
#define KVQ_FMT_Q6     6
#define KVQ_FMT_Q8     8
#define KVQ_FMT_FP16  16   /* uncompressed fp16 (capacity helper only) */

/* fp16 -> per-tensor formats for K and V in one launch (ExLlamaV2 cache
 * page, Description of fp16_to_fp8 and fp16_to_q_kv, generalised). */
KVQ_API int kvq_fp16_to_kv(const void* k_in, void* k_out, void* k_scales, int fmt_k,
                           const void* v_in, void* v_out, void* v_scales, int fmt_v,
                           kvq_shape s, int batch_size, int offset, int width,
                           int page_size, const int32_t* cache_seqlens,
                           const int32_t* block_table, int block_table_cols,
                           void* hip_stream);

/* Per-tensor formats -> fp16 for K and V in one launch, over the same rows
 * (ExLlamaV2 cache page, Description of fp8_to_fp16 and q_to_fp16_kv,
 * generalised).  k_in / v_in are the compact caches, k_out / v_out fp16. */
KVQ_API int kvq_kv_to_fp16(const void* k_in, void* k_out, const void* k_scales, int fmt_k,
                           const void* v_in, void* v_out, const void* v_scales, int fmt_v,
                           kvq_shape s, int batch_size, int offset, int width,
                           int page_size, const int32_t* cache_seqlens,
                           const int32_t* block_table, int block_table_cols,
                           void* hip_stream);

/* Full-prefix widen of a paged cache: for every sequence b < batch_size,
 * positions p in [0, min(cache_seqlens[b] + width, max_len)) -- the cached
 * tokens plus `width` just appended, i.e. everything attention reads (the
 * page's Usage section: the cache classes convert during the attention
 * forward pass) -- are converted from the compact caches into the fp16
 * caches at the same physical rows.  Paged only: page_size = dim1; p lives in
 * page block_table[b * block_table_cols + p / dim1], slot p % dim1; positions
 * past the table or with a page outside [0, dim0) are skipped.  max_len
 * bounds the launch (e.g. block_table_cols * dim1); batch_size * max_len rows
 * are enumerated.  Formats and pointers as kvq_kv_to_fp16. */
KVQ_API int kvq_kv_to_fp16_prefix(const void* k_in, void* k_out, const void* k_scales, int fmt_k,
                                  const void* v_in, void* v_out, const void* v_scales, int fmt_v,
                                  kvq_shape s, int batch_size, int width, int max_len,
                                  const int32_t* cache_seqlens, const int32_t* block_table,
                                  int block_table_cols, void* hip_stream);

/* Bytes one token occupies in one cache tensor (K or V) of a format:
 * KVQ_FMT_FP16 2R, KVQ_FMT_FP8 R, Qb R*b/8 + 2*R/32, with R = heads*head_dim
 * -- the capacity arithmetic a planner needs (the unsloth planning page
 * sizes the KV cache per context length and cache type).  Host only.
 * Returns KVQ_ERR_WBITS for an unknown format, KVQ_ERR_SHAPE for
 * non-positive sizes or head_dim % 32 != 0 with a block format. */
KVQ_API int64_t kvq_bytes_per_token(int format, int heads, int head_dim);

/* Static description of a KVQ_* code ("unknown error" for anything else). */
KVQ_API const char* kvq_strerror(int code);

/* Library version as major * 10000 + minor * 100 + patch. */
KVQ_API int kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
