// Host-side reference stream from rocRAND's Philox4x32-10 engine, used only to
// pin the CPU oracle's Philox.  For each query line "seed b g i" on stdin it
// prints the word the engine yields for counter (i >> 2, g, b, 0) and key seed.
// rocRAND's offset fills counter words x, y (offset / 4) and the lane
// (offset % 4); its subsequence fills words z, w.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
    unsigned long long seed, b, g, i;
    while (std::scanf("%llu %llu %llu %llu", &seed, &b, &g, &i) == 4) {
        unsigned long long offset = 4ull * ((g << 32) | (i >> 2)) + (i & 3ull);
        rocrand_device::philox4x32_10_engine eng(seed, b, offset);
        std::printf("%u\n", eng.next());
    }
    return 0;
}
