// Independent pin for the oracle's Philox4x32-10: rocRAND's own implementation of the
// bijection (a library routine shipped with ROCm, source header only). Reads lines of six
// hex words "c0 c1 c2 c3 k0 k1" on stdin and prints the four output words per line.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct Bijection : rocrand_device::philox4x32_10_engine {
    static uint4 apply(uint4 c, uint2 k) { Bijection e; return e.ten_rounds(c, k); }
};

int main() {
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = Bijection::apply(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
