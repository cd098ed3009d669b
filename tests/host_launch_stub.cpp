// Launcher stand-ins for a host-only build of the C ABI (csrc/kvq_api.cpp)
// with the undefined-behaviour sanitizer: the argument validation and the
// host count_match run as built, and any call that would reach a kernel
// launch returns an error instead (the validation tests never get there).
//
// The stand-ins also check what the validation admitted: a launch the real
// launcher would build with more work-items in a grid dimension than a
// dispatch's 32-bit grid size holds aborts the process (K/V calls: at most
// one 64-lane wavefront per row segment of at least 512 elements, the grid
// padded to a multiple of 8 workgroups of 4 waves; 8-bit calls: one thread
// per 8 elements at most).
#include <stdlib.h>

#include "../kv_cache_quantization_kvq_amd/csrc/kvq_internal.h"

namespace kvq {

static int no_device() { return 1; }

static int64_t mul_or_abort(int64_t a, int64_t b) {
    int64_t r;
    if (__builtin_mul_overflow(a, b, &r)) abort();
    return r;
}

static int kv_launch(const QLaunch& a, bool prefix) {
    const int64_t per_seq = prefix ? a.max_len : a.width;
    const int64_t tensors = (a.k_src ? 1 : 0) + (a.v_src ? 1 : 0);
    const int64_t segments = (a.R + 511) / 512;
    const int64_t units = mul_or_abort(mul_or_abort(mul_or_abort(a.batch, per_seq), tensors), segments);
    const int64_t groups = ((units + 3) / 4 + 7) / 8 * 8;
    if (mul_or_abort(groups, 256) >= (INT64_C(1) << 32)) abort();
    return no_device();
}

static int fp8_launch(const Fp8Launch& a) {
    if (a.span_elems / 8 >= (INT64_C(1) << 32)) abort();
    return no_device();
}

int launch_fp16_to_fp8(const Fp8Launch& a, void*) { return fp8_launch(a); }
int launch_fp8_to_fp16(const Fp8Launch& a, void*) { return fp8_launch(a); }
int launch_quant_kv(const QLaunch& a, void*) { return kv_launch(a, false); }
int launch_dequant_kv(const QLaunch& a, void*) { return kv_launch(a, false); }
int launch_fp16_to_kv(const QLaunch& a, void*) { return kv_launch(a, false); }
int launch_kv_to_fp16(const QLaunch& a, void*) { return kv_launch(a, false); }
int launch_kv_to_fp16_prefix(const QLaunch& a, void*) { return kv_launch(a, true); }
int launch_selftest_codes(const uint16_t*, int64_t, const uint16_t*, int64_t, int, bool, uint8_t*, void*) {
    return no_device();
}
int launch_selftest_scales(const uint16_t*, int64_t, int, uint16_t*, void*) { return no_device(); }
int launch_selftest_fastdiv(const uint32_t*, int64_t, uint32_t, uint32_t*, void*) { return no_device(); }
int launch_selftest_copy(const void*, void*, int64_t n16, int, int, int64_t, void*) {
    if (n16 >= (INT64_C(1) << 32)) abort();
    return no_device();
}
int launch_selftest_stream(const void*, void*, int64_t tiles, int, int group_waves, bool, void*) {
    if (mul_or_abort((tiles + group_waves - 1) / group_waves * group_waves, 64) >= (INT64_C(1) << 32)) abort();
    return no_device();
}

}  // namespace kvq
