// Host check of the multiply-shift divider constants (make_fastdiv in
// kvq_internal.h): (mulhi(n, mul) + n) >> shift == n / d for numerators
// below 2^31, against integer division.  Built and run by tests/test_abi.py.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "kvq_internal.h"

static uint32_t split(uint32_t n, kvq::FastDiv f) {
    const uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
    return (hi + n) >> f.shift;
}

int main() {
    const uint32_t top = 0x7FFFFFFFu;
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 65536; ++d) ds.push_back(d);
    for (int k = 17; k <= 31; ++k) {
        ds.push_back((1u << k) - 1);
        if (k < 31) { ds.push_back(1u << k); ds.push_back((1u << k) + 1); }
    }
    std::mt19937_64 rng(5150);
    for (int i = 0; i < 2000; ++i) ds.push_back((uint32_t)(rng() % top) + 1);
    uint64_t checks = 0;
    for (uint32_t d : ds) {
        const kvq::FastDiv f = kvq::make_fastdiv(d);
        auto check = [&](uint64_t n) {
            if (n > top) return true;
            ++checks;
            return split((uint32_t)n, f) == (uint32_t)n / d;
        };
        bool ok = check(0) && check(1) && check(top) && check(top - 1);
        for (uint64_t m = 1; ok && m <= 64; ++m) ok = check(m * d - 1) && check(m * d) && check(m * d + 1);
        const uint64_t qmax = top / d;                       // the last multiples below 2^31
        for (uint64_t m = qmax > 64 ? qmax - 64 : 1; ok && m <= qmax; ++m)
            ok = check(m * d - 1) && check(m * d) && check(m * d + 1);
        for (int i = 0; ok && i < 64; ++i) ok = check(rng() & top);
        if (!ok) {
            printf("fastdiv mismatch for d = %u\n", d);
            return 1;
        }
    }
    printf("fastdiv ok: %zu divisors, %llu checks\n", ds.size(), (unsigned long long)checks);
    return 0;
}
