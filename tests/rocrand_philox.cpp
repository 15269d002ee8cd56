// Prints Philox-4x32-10 blocks computed by rocRAND's philox4x32_10_engine (a
// library implementation of the generator of Salmon et al., SC'11), used by
// the CPU tests to pin the oracle's Philox constants against an independent
// implementation. Input lines: "seed counter_lo64 counter_hi64" (decimal);
// output lines: the four 32-bit words of philox(counter, key = seed), hex.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
    unsigned long long seed, lo, hi;
    while (std::scanf("%llu %llu %llu", &seed, &lo, &hi) == 3) {
        // subsequence s sets counter words 2..3 to s; an offset of 4c sets
        // words 0..1 to c (four words per counter value)
        rocrand_device::philox4x32_10_engine e(seed, hi, 4ull * lo);
        const unsigned a = e.next(), b = e.next(), c = e.next(), d = e.next();
        std::printf("%08x %08x %08x %08x\n", a, b, c, d);
    }
    return 0;
}
