// Launcher stand-ins for a host-only build of the C ABI (csrc/kvq_api.cpp)
// with the undefined-behaviour sanitizer: the argument validation and the
// host count_match run as built, and any call that would reach a kernel
// launch returns an error instead (the validation tests never get there).
#include "../kv_cache_quantization_kvq_amd/csrc/kvq_internal.h"

namespace kvq {

static int no_device() { return 1; }

int launch_fp16_to_fp8(const Fp8Launch&, void*) { return no_device(); }
int launch_fp8_to_fp16(const Fp8Launch&, void*) { return no_device(); }
int launch_quant_kv(const QLaunch&, void*) { return no_device(); }
int launch_dequant_kv(const QLaunch&, void*) { return no_device(); }
int launch_fp16_to_kv(const QLaunch&, void*) { return no_device(); }
int launch_kv_to_fp16(const QLaunch&, void*) { return no_device(); }
int launch_kv_to_fp16_prefix(const QLaunch&, void*) { return no_device(); }
int launch_selftest_codes(const uint16_t*, int64_t, const uint16_t*, int64_t, int, bool, uint8_t*, void*) {
    return no_device();
}
int launch_selftest_scales(const uint16_t*, int64_t, int, uint16_t*, void*) { return no_device(); }
int launch_selftest_fastdiv(const uint32_t*, int64_t, uint32_t, uint32_t*, void*) { return no_device(); }

}  // namespace kvq
