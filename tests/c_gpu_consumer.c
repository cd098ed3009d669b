/* A C program that drives the conversions through include/kvq.h alone: device
 * memory and a stream from the HIP runtime's C API, no Python and no torch.
 * Each result is compared byte for byte with the oracle's C functions (the
 * test links libkvq_oracle.so and declares the few functions it calls).
 *
 * Cases: paged Q4, Q6 and Q8 round trips (K and V in one call each way) on
 * a paged cache whose table holds an invalid entry, a page outside the cache
 * and positions past the table, with a row length of 192 elements (a partial
 * row segment); then contiguous fp16 -> 8-bit -> fp16.  Output buffers start
 * as sentinel bytes on both sides, so untouched bytes are compared too.
 *
 * Exit status: 0 all equal, 1 a mismatch, 2 an entry point returned an
 * error, 3 a HIP runtime call failed.  Built and run by
 * tests/test_gpu_c_consumer.py. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvq.h"

/* oracle (oracle/kvq_oracle.c) */
void orc_fp16_to_q_kv(const uint16_t* k_in, uint8_t* k_out, uint16_t* k_scales,
                      const uint16_t* v_in, uint8_t* v_out, uint16_t* v_scales,
                      int dim0, int dim1, int heads, int head_dim,
                      int batch_size, int offset, int width, int page_size,
                      const int32_t* cache_seqlens, const int32_t* block_table,
                      int bt_cols, int wbits);
void orc_q_to_fp16_kv(const uint8_t* k_in, uint16_t* k_out, const uint16_t* k_scales,
                      const uint8_t* v_in, uint16_t* v_out, const uint16_t* v_scales,
                      int dim0, int dim1, int heads, int head_dim,
                      int batch_size, int offset, int width, int page_size,
                      const int32_t* cache_seqlens, const int32_t* block_table,
                      int bt_cols, int wbits);
void orc_fp16_to_fp8_cache(const uint16_t* in, uint8_t* out, int dim0, int dim1,
                           int heads, int head_dim, int batch_size, int offset, int width);
void orc_fp8_to_fp16_cache(const uint8_t* in, uint16_t* out, int dim0, int dim1,
                           int heads, int head_dim, int batch_size, int offset, int width);

#define SENTINEL 0xA5

#define HIP(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) { \
    fprintf(stderr, "HIP error %d at line %d: %s\n", (int)e_, __LINE__, #call); exit(3); } } while (0)
#define KVQ(call) do { int r_ = (call); if (r_ != KVQ_OK) { \
    fprintf(stderr, "kvq error %d (%s) at line %d: %s\n", r_, kvq_strerror(r_), __LINE__, #call); exit(2); } } while (0)

static int failures = 0;

static void compare(const char* what, const void* gpu, const void* ref, size_t n)
{
    const uint8_t* a = (const uint8_t*)gpu;
    const uint8_t* b = (const uint8_t*)ref;
    for (size_t i = 0; i < n; ++i)
        if (a[i] != b[i]) {
            fprintf(stderr, "%s: first difference at byte %zu (gpu %#x, oracle %#x)\n", what, i, a[i], b[i]);
            ++failures;
            return;
        }
}

/* device copy of a host buffer */
static void* upload(const void* h, size_t n)
{
    void* d = NULL;
    HIP(hipMalloc(&d, n));
    HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

/* device buffer filled with the sentinel */
static void* sentinel_buffer(size_t n)
{
    void* d = NULL;
    HIP(hipMalloc(&d, n));
    HIP(hipMemset(d, SENTINEL, n));
    return d;
}

static void* host_sentinel(size_t n)
{
    void* h = malloc(n);
    if (!h) exit(3);
    memset(h, SENTINEL, n);
    return h;
}

static void* download(const void* d, size_t n)
{
    void* h = malloc(n);
    if (!h) exit(3);
    HIP(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
    return h;
}

/* finite fp16 bits with magnitudes between 2^-10 and 2^6 */
static uint32_t lcg_state = 12345u;
static uint16_t next_f16(void)
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    const uint32_t r = lcg_state >> 8;
    const uint16_t sign = (uint16_t)((r & 1u) << 15);
    const uint16_t expo = (uint16_t)(5u + (r >> 1) % 16u);
    const uint16_t mant = (uint16_t)((r >> 5) & 0x3FFu);
    return (uint16_t)(sign | (expo << 10) | mant);
}

int main(void)
{
    /* 12 pages of 16 tokens, 2 heads x 96: 192 elements per token row */
    const kvq_shape s = {12, 16, 2, 96};
    const int R = s.heads * s.head_dim;
    const size_t rows = (size_t)s.dim0 * s.dim1;
    const size_t n_f16 = rows * (size_t)R * 2;
    const size_t n_sc = rows * (size_t)(R / 32) * 2;

    /* three sequences, four table columns: an invalid entry (-1), a page
     * outside the cache (12), and positions 64.. past the table */
    const int batch = 3, cols = 4, width = 20;
    const int32_t bt[12] = {3, 7, -1, 11, 0, 12, 5, 9, 2, 4, 6, 8};
    const int32_t sl[3] = {0, 5, 50};

    uint16_t* k = (uint16_t*)malloc(n_f16);
    uint16_t* v = (uint16_t*)malloc(n_f16);
    if (!k || !v) return 3;
    for (size_t i = 0; i < rows * (size_t)R; ++i) {
        k[i] = next_f16();
        v[i] = next_f16();
    }
    for (int i = 0; i < 32; ++i) k[3 * 16 * R + i] = 0;     /* an all-zero block in page 3, row 0 */

    int ndev = 0;
    HIP(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        fprintf(stderr, "no HIP device\n");
        return 3;
    }
    hipStream_t stream;
    HIP(hipStreamCreate(&stream));
    void* dk = upload(k, n_f16);
    void* dv = upload(v, n_f16);
    void* dsl = upload(sl, sizeof sl);
    void* dbt = upload(bt, sizeof bt);

    const int widths[3] = {4, 6, 8};
    for (int w = 0; w < 3; ++w) {
        const int wb = widths[w];
        const size_t n_code = rows * (size_t)R * wb / 8;
        void* dkq = sentinel_buffer(n_code);
        void* dvq = sentinel_buffer(n_code);
        void* dks = sentinel_buffer(n_sc);
        void* dvs = sentinel_buffer(n_sc);
        void* dko = sentinel_buffer(n_f16);
        void* dvo = sentinel_buffer(n_f16);
        KVQ(kvq_fp16_to_q_kv(dk, dkq, dks, dv, dvq, dvs, s, batch, 0, width, s.dim1,
                             (const int32_t*)dsl, (const int32_t*)dbt, cols, wb, stream));
        KVQ(kvq_q_to_fp16_kv(dkq, dko, dks, dvq, dvo, dvs, s, batch, 0, width, s.dim1,
                             (const int32_t*)dsl, (const int32_t*)dbt, cols, wb, stream));
        HIP(hipStreamSynchronize(stream));

        uint8_t* okq = (uint8_t*)host_sentinel(n_code);
        uint8_t* ovq = (uint8_t*)host_sentinel(n_code);
        uint16_t* oks = (uint16_t*)host_sentinel(n_sc);
        uint16_t* ovs = (uint16_t*)host_sentinel(n_sc);
        uint16_t* oko = (uint16_t*)host_sentinel(n_f16);
        uint16_t* ovo = (uint16_t*)host_sentinel(n_f16);
        orc_fp16_to_q_kv(k, okq, oks, v, ovq, ovs, s.dim0, s.dim1, s.heads, s.head_dim,
                         batch, 0, width, s.dim1, sl, bt, cols, wb);
        orc_q_to_fp16_kv(okq, oko, oks, ovq, ovo, ovs, s.dim0, s.dim1, s.heads, s.head_dim,
                         batch, 0, width, s.dim1, sl, bt, cols, wb);

        const void* dev_bufs[6] = {dkq, dks, dvq, dvs, dko, dvo};
        const void* ref_bufs[6] = {okq, oks, ovq, ovs, oko, ovo};
        const size_t sizes[6] = {n_code, n_sc, n_code, n_sc, n_f16, n_f16};
        const char* names[6] = {"K codes", "K scales", "V codes", "V scales", "K out", "V out"};
        for (int i = 0; i < 6; ++i) {
            char what[64];
            void* got = download(dev_bufs[i], sizes[i]);
            snprintf(what, sizeof what, "paged Q%d %s", wb, names[i]);
            compare(what, got, ref_bufs[i], sizes[i]);
            free(got);
        }
        free(okq); free(ovq); free(oks); free(ovs); free(oko); free(ovo);
        HIP(hipFree(dkq)); HIP(hipFree(dvq)); HIP(hipFree(dks)); HIP(hipFree(dvs));
        HIP(hipFree(dko)); HIP(hipFree(dvo));
    }

    /* contiguous 8-bit: the same fp16 data read as [12, 16, 2, 96] with
     * batch 10, window 3 .. 15 */
    {
        const size_t n8 = rows * (size_t)R;
        void* d8 = sentinel_buffer(n8);
        void* dback = sentinel_buffer(n_f16);
        KVQ(kvq_fp16_to_fp8(dk, d8, s, 10, 3, 12, stream));
        KVQ(kvq_fp8_to_fp16(d8, dback, s, 10, 3, 12, stream));
        HIP(hipStreamSynchronize(stream));
        uint8_t* o8 = (uint8_t*)host_sentinel(n8);
        uint16_t* oback = (uint16_t*)host_sentinel(n_f16);
        orc_fp16_to_fp8_cache(k, o8, s.dim0, s.dim1, s.heads, s.head_dim, 10, 3, 12);
        orc_fp8_to_fp16_cache(o8, oback, s.dim0, s.dim1, s.heads, s.head_dim, 10, 3, 12);
        void* g8 = download(d8, n8);
        void* gback = download(dback, n_f16);
        compare("contiguous 8-bit", g8, o8, n8);
        compare("contiguous 8-bit back to fp16", gback, oback, n_f16);
        free(g8); free(gback); free(o8); free(oback);
        HIP(hipFree(d8)); HIP(hipFree(dback));
    }

    HIP(hipFree(dk)); HIP(hipFree(dv)); HIP(hipFree(dsl)); HIP(hipFree(dbt));
    HIP(hipStreamDestroy(stream));
    free(k);
    free(v);
    if (failures) return 1;
    printf("c gpu consumer ok\n");
    return 0;
}
