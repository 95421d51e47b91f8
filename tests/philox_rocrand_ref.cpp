// Second, independent Philox4x32-10: rocRAND's host-callable engine.  Used only
// by the oracle's pin test.  Reads "seed subsequence offset" triples on stdin
// and prints the four 32-bit words rocRAND returns after skipping to that
// (subsequence, offset): counter = (offset/4 as 64 bits, subsequence as 64
// bits), key = seed.
#include <cstdio>
#include <rocrand/rocrand_kernel.h>

int main() {
    unsigned long long seed, subseq, offset;
    while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, subseq, offset, &st);
        uint4 w = rocrand4(&st);
        std::printf("%u %u %u %u\n", w.x, w.y, w.z, w.w);
    }
    return 0;
}
