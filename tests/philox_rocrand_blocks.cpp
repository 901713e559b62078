// Prints raw Philox4x32-10 blocks computed by rocRAND's host-callable engine,
// for (counter, key) lines read from stdin ("c0 c1 c2 c3 k0 k1" in hex).
// Used by the CPU tests as an implementation of Philox independent of the
// oracle's.  Host code only; nothing runs on a GPU.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

struct RawPhilox : rocrand_device::philox4x32_10_engine {
    uint4 block(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};

int main() {
    RawPhilox eng;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = eng.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
