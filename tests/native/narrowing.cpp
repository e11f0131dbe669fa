// Host check of the exact search's range arithmetic (wave_select.h): for
// every level-1 bin, the widest sub-range each narrowing pass can leave is
// followed down to a single key value; the pass count must stay within
// NARROW_PASSES and every pass must fit its histogram.
#include <cstdio>
#include <cstdint>
#include "wave_select.h"

int main() {
    using namespace csa;
    int worst = 0;
    for (int d = 0; d < SEL_NB; ++d) {
        uint32_t lo, hi;
        lvl1_range(d, &lo, &hi);
        if (hi <= lo) { std::printf("bin %d: empty range\n", d); return 1; }
        // keys of bin d are exactly [lo, hi)
        if (lvl1_bin(lo) != d || (hi != KEY_END && lvl1_bin(hi) != d + 1) ||
            lvl1_bin(hi - 1u) != d) {
            std::printf("bin %d: range [%u, %u) disagrees with lvl1_bin\n", d, lo, hi);
            return 1;
        }
        int passes = 0;
        while (hi - lo > 1u) {
            const int sh = range_shift(lo, hi);
            const uint64_t nbins = ((uint64_t)(hi - lo - 1u) >> sh) + 1u;
            if (nbins > (uint64_t)SEL_NB) {
                std::printf("bin %d: %llu sub-ranges\n", d, (unsigned long long)nbins);
                return 1;
            }
            // the widest sub-range is a whole one (the last may be clamped)
            const uint64_t top = (uint64_t)lo + (1ull << sh);
            hi = top < (uint64_t)hi ? (uint32_t)top : hi;
            ++passes;
        }
        if (passes > worst) worst = passes;
    }
    std::printf("worst narrowing passes %d bound %d exact passes %d\n", worst, NARROW_PASSES,
                EXACT_PASSES);
    return worst <= NARROW_PASSES ? 0 : 1;
}
