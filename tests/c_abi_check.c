/* Plain C99 consumer of include/kvq.h and include/kvq_selftest.h: the
 * headers compile as C and the host-side entry points behave as declared.
 * Built and run by tests/test_abi.py; no GPU call is made (every device
 * entry point below is rejected by its host-side validation). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvq.h"
#include "kvq_selftest.h"

static int failures = 0;
#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "FAILED: %s (line %d)\n", #cond, __LINE__); ++failures; } } while (0)

int main(void)
{
    int32_t a[10] = {1, 2, 3, 4, 5, 6, 7, 8, 9, 10};
    int32_t b[10] = {1, 2, 3, 4, 5, 6, 0, 8, 9, 10};
    int64_t x[3] = {7, 8, 9};
    kvq_shape s = {4, 16, 2, 64};
    kvq_shape bad = {4, 16, 2, 48};
    void* p = (void*)(uintptr_t)0x7F0000000000ull;      /* never dereferenced */
    void* q = (void*)(uintptr_t)0x7F0040000000ull;

    CHECK(kvq_version() >= 100);
    CHECK(strcmp(kvq_strerror(KVQ_OK), "success") == 0);
    CHECK(strcmp(kvq_strerror(-99), "unknown error") == 0);

    CHECK(kvq_count_match(a, 10, b, 10, 10, 4) == 6);
    CHECK(kvq_count_match(a, 10, b, 10, 4, 4) == 4);
    CHECK(kvq_count_match(a, 10, a, 10, 100, 4) == 10);
    CHECK(kvq_count_match(x, 3, x, 3, 3, 8) == 3);
    CHECK(kvq_count_match(a, 10, b, 10, 10, 2) == KVQ_ERR_RANGE);

    CHECK(kvq_bytes_per_token(KVQ_FMT_FP16, 8, 128) == 2048);
    CHECK(kvq_bytes_per_token(KVQ_FMT_FP8, 8, 128) == 1024);
    CHECK(kvq_bytes_per_token(KVQ_FMT_Q4, 8, 128) == 576);
    CHECK(kvq_bytes_per_token(KVQ_FMT_Q6, 8, 128) == 832);
    CHECK(kvq_bytes_per_token(KVQ_FMT_Q8, 8, 128) == 1088);
    CHECK(kvq_bytes_per_token(5, 8, 128) == KVQ_ERR_WBITS);

    /* validation only: each call fails before anything is enqueued */
    CHECK(kvq_fp16_to_q_kv(p, q, NULL, NULL, NULL, NULL, s, 1, 0, 4, 0, NULL, NULL, 0, 4, NULL) == KVQ_ERR_NULL);
    CHECK(kvq_fp16_to_q_kv(p, q, p, NULL, NULL, NULL, s, 1, 0, 4, 0, NULL, NULL, 0, 5, NULL) == KVQ_ERR_WBITS);
    CHECK(kvq_q_to_fp16_kv(p, q, p, NULL, NULL, NULL, bad, 1, 0, 4, 0, NULL, NULL, 0, 4, NULL) == KVQ_ERR_SHAPE);
    CHECK(kvq_fp16_to_fp8(p, q, s, 5, 0, 4, NULL) == KVQ_ERR_RANGE);
    CHECK(kvq_fp8_to_fp16(p, (char*)q + 4, s, 1, 0, 4, NULL) == KVQ_ERR_ALIGN);
    CHECK(kvq_fp16_to_kv(p, p, NULL, KVQ_FMT_FP8, NULL, NULL, NULL, 0, s, 1, 0, 4, 0, NULL, NULL, 0, NULL)
          == KVQ_ERR_OVERLAP);
    CHECK(kvq_kv_to_fp16(p, q, NULL, 3, NULL, NULL, NULL, 0, s, 1, 0, 4, 0, NULL, NULL, 0, NULL) == KVQ_ERR_WBITS);
    CHECK(kvq_kv_to_fp16_prefix(p, q, NULL, KVQ_FMT_FP8, NULL, NULL, NULL, 0, s, 1, 2, 8, NULL, NULL, 4, NULL)
          == KVQ_ERR_NULL);
    CHECK(kvq_selftest_fastdiv((const uint32_t*)p, 4, 0, (uint32_t*)q, NULL) == KVQ_ERR_RANGE);
    CHECK(kvq_selftest_scales((const uint16_t*)p, 4, 5, (uint16_t*)q, NULL) == KVQ_ERR_WBITS);
    CHECK(kvq_selftest_copy(p, q, 1000, 16, 1, 0, NULL) == KVQ_ERR_RANGE);
    CHECK(kvq_selftest_stream(p, 4096, q, 2048, 4, 1, NULL) == KVQ_ERR_RANGE);
    CHECK(kvq_selftest_stream(p, 0, q, 0, 4, 1, NULL) == KVQ_OK);

    /* zero work validates and returns without a launch */
    CHECK(kvq_fp16_to_q_kv(p, q, (char*)q + (1 << 24), NULL, NULL, NULL, s, 0, 0, 4, 0, NULL, NULL, 0, 4, NULL)
          == KVQ_OK);

    if (failures) return 1;
    printf("c abi ok\n");
    return 0;
}
