// Host check of the launch-invariant division used by the tile walk and the
// row decode: FastDiv::div(n) against n / d for every divisor 1..70000 and a
// spread of larger ones, on quotient boundaries and pseudo-random numerators
// below 2^31. Prints the number of mismatches (0 expected) and exits with 1 on any.
#include "igconv_internal.h"

#include <cstdio>
#include <cstdint>

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next31()
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 33);
}

int main()
{
    long long bad = 0, checks = 0;
    auto check = [&](const igc::FastDiv &f, long long d, long long n) {
        if (n < 0 || n > 0x7fffffffll)
            return;
        ++checks;
        if (f.div((int)n) != n / d) {
            if (bad < 10)
                std::printf("d=%lld n=%lld got %d want %lld\n", d, n, f.div((int)n), n / d);
            ++bad;
        }
    };
    auto divisor = [&](long long d) {
        igc::FastDiv f;
        f.set(d);
        const long long top = 0x7fffffffll / d;
        for (long long k : {0ll, 1ll, 2ll, 3ll, top / 2, top - 1, top, top + 1}) {
            check(f, d, k * d - 1);
            check(f, d, k * d);
            check(f, d, k * d + d - 1);
        }
        check(f, d, 0x7fffffffll);
        for (int i = 0; i < 16; ++i)
            check(f, d, next31());
    };
    for (long long d = 1; d <= 70000; ++d)
        divisor(d);
    for (int s = 17; s <= 31; ++s)
        for (long long d : {(1ll << s) - 1, 1ll << s, (1ll << s) + 1, (3ll << (s - 1)) + 7})
            if (d <= 0x7fffffffll)
                divisor(d);
    for (int i = 0; i < 20000; ++i)
        divisor(1 + next31());
    std::printf("%lld checks, %lld mismatches\n", checks, bad);
    return bad ? 1 : 0;
}
