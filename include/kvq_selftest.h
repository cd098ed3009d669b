/*
 * kvq_selftest.h -- verification hooks of the kvq library.
 *
 * They run the exact device routines the conversion kernels use (scale rule,
 * per-element code computation) on caller-chosen operands, so a test can
 * sweep every fp16 (x, scale) pair against an independent reference.  The
 * arithmetic they expose is the block quantization of the ExLlamaV2 cache
 * page (Description of fp16_to_q_kv; I/O Contract: per-block scale factors,
 * wbits 4 or 6, plus 8 here) with the numeric reading stated in kvq.h, and
 * the row split of the paged addressing (Description: block_table /
 * cache_seqlens).
 * Same conventions as kvq.h: device pointers, asynchronous on hip_stream,
 * 0 or a negative KVQ_ERR_* code.
 */
#ifndef KVQ_SELFTEST_H
#define KVQ_SELFTEST_H

#include <stdint.h>

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * u_out[i * nx + j] = offset-binary code (one per byte) of fp16 x[j] under
 * the stored fp16 scale s16[i], for i < ns, j < nx.
 *   x      device, fp16 bits [nx], nx % 8 == 0, 16-byte aligned
 *   s16    device, fp16 bits [ns] (scales >= 0; 0 gives the zero code)
 *   u_out  device, uint8 [ns, nx], 16-byte aligned
 *   force_clamp  0: the kernels' own dispatch -- the clamp to
 *                [-2^(b-1), 2^(b-1)-1] is applied only for subnormal scales,
 *                which is exact whenever |x / s16| < 2^(b-1) - 1/2 (always
 *                true for elements of the block a normal scale came from);
 *                pairs outside that domain under a normal scale give an
 *                unspecified code in this mode.
 *                1: always take the clamping path (defined on every pair).
 */
KVQ_API int kvq_selftest_codes(const uint16_t* x, int64_t nx, const uint16_t* s16, int64_t ns,
                               int wbits, int force_clamp, uint8_t* u_out, void* hip_stream);

/*
 * out[i] = stored fp16 scale of a block whose absmax is the fp16 absmax[i]
 * (>= 0, finite).  Device pointers, 2-byte aligned.
 */
KVQ_API int kvq_selftest_scales(const uint16_t* absmax, int64_t n, int wbits, uint16_t* out,
                        void* hip_stream);

/*
 * q[i] = n[i] / d (integer division) through the multiply-shift divider the
 * kernels use to split logical rows into (sequence, token) and positions
 * into (page, slot).  n[i] < 2^31, 1 <= d < 2^31; device pointers, 4-byte
 * aligned.  KVQ_ERR_RANGE for d or count out of range.
 */
KVQ_API int kvq_selftest_fastdiv(const uint32_t* n, int64_t count, uint32_t d, uint32_t* q,
                                 void* hip_stream);

/*
 * dst[0 .. bytes) = src[0 .. bytes) by a plain non-temporal copy kernel: the
 * bandwidth reference the conversions are measured against (one launch of a
 * given size, no conversion work).  A wave moves tiles of lane_bytes x 64
 * bytes (lane_bytes / 16 loads of 16 bytes per lane, all issued before its
 * stores); workgroups hold group_waves waves; with max_waves > 0 at most that
 * many waves run and stride over the tiles, otherwise one wave per tile.
 *   src, dst     device, 16-byte aligned, non-overlapping
 *   bytes        >= 0, a multiple of 16
 *   lane_bytes   16, 32, 64 or 128;  group_waves 1, 2, 4 or 8
 * KVQ_ERR_RANGE / _ALIGN / _OVERLAP / _NULL before anything is enqueued.
 */
KVQ_API int kvq_selftest_copy(const void* src, void* dst, int64_t bytes, int lane_bytes, int group_waves,
                              int64_t max_waves, void* hip_stream);

/*
 * Bandwidth reference for uneven traffic, the shapes of the conversions
 * (quantize reads about 3.6 bytes per byte written, dequantize the
 * reverse): per tile of 64 lanes x 16 bytes on the light side, each lane
 * reads (gather) or writes (scatter) lane_elems 16-byte elements on the
 * heavy side.  Gather: src_bytes == lane_elems * dst_bytes, and light
 * element i of dst is the XOR of src elements (i / 64) * 64 * lane_elems +
 * 64 k + i % 64, k < lane_elems.  Scatter: dst_bytes == lane_elems *
 * src_bytes, and those dst elements all equal src element i.  All loads
 * and stores are non-temporal; one wave per tile, group_waves per
 * workgroup.
 *   src, dst      device, 16-byte aligned, non-overlapping
 *   light side    a multiple of 1024 bytes; both sizes below 2^56
 *   lane_elems    2, 4 or 8;  group_waves 1, 2, 4 or 8
 * KVQ_ERR_RANGE (sizes not in one of the two ratios, or out of range) /
 * _ALIGN / _OVERLAP / _NULL before anything is enqueued; zero sizes launch
 * nothing.
 */
KVQ_API int kvq_selftest_stream(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                                int lane_elems, int group_waves, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_SELFTEST_H */
