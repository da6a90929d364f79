// Host check of the launch-time divisor (FastDiv): fdiv(n, make_fastdiv(d))
// must equal n / d for every dividend below 2^31.  Covers every divisor
// below 70000 at multiples of d and their neighbours, the largest
// dividends, and random divisors and dividends over the whole range.
// Prints the number of mismatches; exit status 1 if any.
#include "../../cnn_convolution_lowering_amd/csrc/device_common.hpp"

#include <cstdio>
#include <random>

using convlower::FastDiv;
using convlower::fdiv;
using convlower::make_fastdiv;

int main() {
    std::mt19937_64 rng(7);
    long checked = 0, bad = 0;
    auto check = [&](uint32_t n, const FastDiv& f) {
        ++checked;
        if (fdiv(n, f) != n / f.d) {
            if (bad < 5) std::printf("mismatch: n=%u d=%u\n", n, f.d);
            ++bad;
        }
    };
    for (uint32_t d = 1; d < 70000; ++d) {
        const FastDiv f = make_fastdiv(d);
        for (uint64_t k : {0ull, 1ull, 2ull, 3ull, 1000ull}) {
            for (int o = -1; o <= 1; ++o) {
                const int64_t n = int64_t(k * d) + o;
                if (n >= 0 && n < (int64_t(1) << 31)) check(uint32_t(n), f);
            }
        }
        check(0x7fffffffu, f);
        check(0x7ffffffeu, f);
        for (int i = 0; i < 20; ++i) check(uint32_t(rng() & 0x7fffffffu), f);
    }
    for (int i = 0; i < 100000; ++i) {
        const uint32_t d = uint32_t(rng() % 0x7fffffffu) + 1;
        const FastDiv f = make_fastdiv(d);
        check(d - 1, f);
        check(d, f);
        check(0x7fffffffu, f);
        for (int k = 0; k < 10; ++k) check(uint32_t(rng() & 0x7fffffffu), f);
    }
    std::printf("checked %ld mismatches %ld\n", checked, bad);
    return bad != 0;
}
