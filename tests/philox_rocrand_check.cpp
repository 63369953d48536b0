// Reads lines "key0 key1 c0 c1 c2 c3" (hex) and prints the four output words
// of rocRAND's Philox4x32-10 block function for that key and counter.  A
// library implementation of Philox4x32-10, used to pin the oracle's own
// implementation; host code only.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct philox_block : rocrand_device::philox4x32_10_engine {
    uint4 apply(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};

int main()
{
    unsigned k0, k1, c0, c1, c2, c3;
    philox_block p;
    while (std::scanf("%x %x %x %x %x %x", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        uint4 ctr;
        ctr.x = c0; ctr.y = c1; ctr.z = c2; ctr.w = c3;
        uint2 key;
        key.x = k0; key.y = k1;
        uint4 r = p.apply(ctr, key);
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
