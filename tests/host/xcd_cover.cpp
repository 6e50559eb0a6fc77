// Host check of the XCD-aware block remap of the grouped GEMM launches: for a
// grid of xcd_grid(items) blocks, every logical tile L < n_valid (any
// n_valid <= items) is reached by exactly one block and no block gets a tile
// past n_valid.  Built with hipcc as host code and run on the CPU.
#include <cstdio>
#include <vector>

#include "../../expert_layer_amd/csrc/common.hpp"

int main() {
    long checked = 0;
    for (int items = 0; items <= 700; ++items) {
        const int grid = (int)moe::xcd_grid(items);
        if (grid % 8 || grid < items || grid >= items + 8) {
            std::printf("bad grid %d for %d items\n", grid, items);
            return 1;
        }
        for (int n_valid = 0; n_valid <= items; ++n_valid) {
            std::vector<int> hits(n_valid > 0 ? n_valid : 1, 0);
            for (int b = 0; b < grid; ++b) {
                const int L = moe::xcd_remap(b, n_valid);
                if (L >= n_valid || L < -1) {
                    std::printf("block %d -> %d outside [0, %d)\n", b, L, n_valid);
                    return 1;
                }
                if (L >= 0) ++hits[L];
            }
            for (int L = 0; L < n_valid; ++L)
                if (hits[L] != 1) {
                    std::printf("items %d n_valid %d: tile %d reached %d times\n", items, n_valid, L, hits[L]);
                    return 1;
                }
            ++checked;
        }
    }
    // the run-interleaved remap over xcd_grid_runs(items) blocks
    for (int items = 0; items <= 1300; items += (items < 600 ? 1 : 7)) {
        const int grid = (int)moe::xcd_grid_runs(items);
        if (grid % 256 || grid < items) {
            std::printf("bad run grid %d for %d items\n", grid, items);
            return 1;
        }
        for (int n_valid = 0; n_valid <= items; n_valid += (n_valid < 300 ? 1 : 5)) {
            std::vector<int> hits(n_valid > 0 ? n_valid : 1, 0);
            for (int b = 0; b < grid; ++b) {
                const int L = moe::xcd_remap_runs(b, n_valid);
                if (L >= n_valid || L < -1) {
                    std::printf("runs: block %d -> %d outside [0, %d)\n", b, L, n_valid);
                    return 1;
                }
                if (L >= 0) ++hits[L];
            }
            for (int L = 0; L < n_valid; ++L)
                if (hits[L] != 1) {
                    std::printf("runs: items %d n_valid %d: tile %d reached %d times\n", items, n_valid, L, hits[L]);
                    return 1;
                }
            ++checked;
        }
    }
    // the case of a grid that is not a multiple of 8 leaves tiles out (the
    // reason for xcd_grid): 46 blocks, 42 valid tiles
    int hit41 = 0;
    for (int b = 0; b < 46; ++b) hit41 += moe::xcd_remap(b, 42) == 41;
    std::printf("checked %ld (items, n_valid) pairs; unrounded grid 46 reaches tile 41: %d\n", checked, hit41);
    return hit41 == 0 ? 0 : 2;
}
