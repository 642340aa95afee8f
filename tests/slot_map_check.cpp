// Host check of the grouped GEMM's XCD slot map (launch.hpp): for random
// tile tables, every active (M tile, N tile) pair is taken by exactly one
// block of the launch grid.  Prints "ok <cases>" or the first failure.
#include "launch.hpp"

#include <cstdio>
#include <random>
#include <vector>

static int check(int max_tiles, int tiles, int shared_tiles, int ntn) {
    const int total = tiles * ntn, total_r = (tiles - shared_tiles) * ntn;
    const unsigned grid = moe::job_blocks(max_tiles, ntn);
    std::vector<int> hits(static_cast<size_t>(total), 0);
    for (unsigned b = 0; b < grid; ++b) {
        const int lin = moe::xcd_slot_pair(static_cast<int>(b), total_r, total);
        if (lin < -1 || lin >= total) {
            std::printf("FAIL max_tiles=%d tiles=%d shared=%d ntn=%d block %u -> %d\n", max_tiles, tiles,
                        shared_tiles, ntn, b, lin);
            return 1;
        }
        if (lin >= 0) ++hits[static_cast<size_t>(lin)];
    }
    for (int i = 0; i < total; ++i) {
        if (hits[static_cast<size_t>(i)] != 1) {
            std::printf("FAIL max_tiles=%d tiles=%d shared=%d ntn=%d pair %d taken %d times\n", max_tiles, tiles,
                        shared_tiles, ntn, i, hits[static_cast<size_t>(i)]);
            return 1;
        }
    }
    return 0;
}

int main() {
    std::mt19937 rng(12345);
    int cases = 0;
    // exhaustive small tables, then random large ones (up to K2 prefill
    // scale: 1408 M tiles of 14 N tiles)
    for (int max_tiles = 0; max_tiles <= 40; ++max_tiles)
        for (int tiles = 0; tiles <= max_tiles; ++tiles)
            for (int sh = 0; sh <= tiles; ++sh)
                for (int ntn : {1, 2, 3, 8, 14}) {
                    if (check(max_tiles, tiles, sh, ntn)) return 1;
                    ++cases;
                }
    for (int i = 0; i < 20000; ++i) {
        const int max_tiles = 1 + static_cast<int>(rng() % 1500);
        const int tiles = static_cast<int>(rng() % (max_tiles + 1));
        const int sh = static_cast<int>(rng() % (tiles + 1));
        const int ntn = 1 + static_cast<int>(rng() % 16);
        if (check(max_tiles, tiles, sh, ntn)) return 1;
        ++cases;
    }
    std::printf("ok %d\n", cases);
    return 0;
}
