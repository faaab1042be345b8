// Reference Philox4x32-10 words from rocRAND's public engine, used by the CPU
// tests to pin the oracle's own Philox against an independent library.
// Reads lines "key_lo key_hi c0 c1 c2 c3" (decimal) on stdin and prints the
// four 32-bit output words of that counter block.
//
// rocRAND's engine keys itself with the 64-bit seed (low word first) and sets
// counter words 0-1 from offset/4 and words 2-3 from the subsequence, so
// seed(key, subsequence = c2 | c3<<32, offset = 4*(c0 | c1<<32)) positions it
// on counter (c0, c1, c2, c3); the next four draws are that block's words.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdint>

int main()
{
    unsigned long long klo, khi, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu %llu", &klo, &khi, &c0, &c1, &c2, &c3) == 6) {
        unsigned long long seed = (khi << 32) | klo;
        unsigned long long sub = (c3 << 32) | c2;
        unsigned long long off = ((c1 << 32) | c0) * 4ull;
        rocrand_device::philox4x32_10_engine eng(seed, sub, off);
        unsigned int w[4];
        for (int i = 0; i < 4; ++i) w[i] = eng();
        std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
    }
    return 0;
}
