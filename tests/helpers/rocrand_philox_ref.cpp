// Host-side reference: prints rocRAND's Philox4x32-10 block function for the
// counters/keys read from stdin ("c0 c1 c2 c3 k0 k1" in hex per line).  Used
// by the oracle's Philox pin; it runs rocRAND's header code on the CPU only.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

struct block_fn : rocrand_device::philox4x32_10_engine {
    uint4 operator()(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};

int main() {
    block_fn fn;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = fn(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
