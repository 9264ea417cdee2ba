// Host-side driver for rocRAND's Philox4x32-10 block function, used only as
// an independent pin for the oracle's Philox implementation.
//
// Reads lines "k0 k1 c0 c1 c2 c3" (decimal) from stdin and prints the four
// 32-bit output words of the ten-round block function for that key and
// counter.  The engine keeps the block function protected, so a derived
// class exposes it.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

struct philox_block : rocrand_device::philox4x32_10_engine {
    uint4 eval(uint4 counter, uint2 key) { return ten_rounds(counter, key); }
};

int main() {
    unsigned int k0, k1, c0, c1, c2, c3;
    philox_block blk;
    while (std::scanf("%u %u %u %u %u %u", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        uint4 r = blk.eval(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
