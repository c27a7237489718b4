// Reference Philox4x32-10 outputs from rocRAND's engine (an independent library
// implementation), used to pin the oracle's Philox on the CPU.
// stdin: lines "seed c0 c1 c2 c3" (decimal; counter words 0..3 with c1 = high
// word of the block index as rocRAND lays it out); stdout: 4 output words.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
        // rocRAND: key = seed; counter = (offset/4 as 64 bits in words 0,1; subsequence in words 2,3)
        unsigned long long subsequence = c2 | (c3 << 32);
        unsigned long long block = c0 | (c1 << 32);
        rocrand_device::philox4x32_10_engine eng(seed, subsequence, 0);
        // advance `block` counter steps by skipping 4*block outputs
        eng.discard(block * 4ULL);
        uint4 r = eng.next4();
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
