// Independent Philox4x32-10 reference for the oracle's pin test: rocRAND's
// header-only engine, compiled for the host with g++.  Reads lines
// "seed subsequence offset" from stdin and prints the four 32-bit words the
// engine yields at that position.  With offset = 4*g the engine's counter is
// (g mod 2^32, g >> 32, subsequence mod 2^32, subsequence >> 32) and its key
// is (seed mod 2^32, seed >> 32).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main()
{
    unsigned long long seed, sub, off;
    while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
        rocrand_device::philox4x32_10_engine e(seed, sub, off);
        uint4 r = e.next4();
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
