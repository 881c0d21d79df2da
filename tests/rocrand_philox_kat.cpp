// Host-only helper for the oracle's generator test: prints Philox4x32-10
// words produced by rocRAND's engine, compiled from its source header.
// Input lines: "seed subsequence offset" (decimal, 64-bit). For each line it
// prints the 32-bit word the engine returns first, in hex. With rocRAND's
// layout that word is word (offset & 3) of the 10-round function applied to
// counter (lo(offset/4), hi(offset/4), lo(subsequence), hi(subsequence)) under
// key (lo(seed), hi(seed)).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, subsequence, offset;
    while (std::scanf("%llu %llu %llu", &seed, &subsequence, &offset) == 3) {
        rocrand_device::philox4x32_10_engine engine(seed, subsequence, offset);
        std::printf("%08x\n", engine());
    }
    return 0;
}
