// Test-only host program: evaluates Philox-4x32-10 with rocRAND's open-source
// header (an implementation independent of this project) for the
// (counter, key) tuples read from stdin, one "c0 c1 c2 c3 k0 k1" per line,
// and prints the four output words per line.  Built and run by the CPU tests.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

struct philox_block : rocrand_device::philox4x32_10_engine {
    uint4 eval(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};

int main() {
    philox_block gen;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 ctr;
        ctr.x = c0; ctr.y = c1; ctr.z = c2; ctr.w = c3;
        uint2 key;
        key.x = k0; key.y = k1;
        uint4 r = gen.eval(ctr, key);
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
