// Host check of the XCD-aware block remap of the grouped GEMM launches: for a
// grid of xcd_grid(items) blocks, every logical tile L < n_valid (any
// n_valid <= items) is reached by exactly one block and no block gets a tile
// past n_valid; the same for the work queues (xcd_queue_pick over
// xcd_queue_grid(items) blocks) whatever order the blocks run in.  Built with
// hipcc as host code and run on the CPU.
#include <algorithm>
#include <cstdio>
#include <random>
#include <vector>

#include "../../expert_layer_amd/csrc/common.hpp"

// The queue's atomic accesses, run one block at a time.
struct HostQueue {
    int c[moe::kQueueWords] = {0};
    int empty() { return c[8]; }
    int draw(int y) { return c[y]++; }
    void mark(int y) { c[8] |= 1 << y; }
};

// Runs the blocks of a queue grid in `order`; returns 0 when every tile is
// taken once, and the tiles each XCD took in `per_xcd`.
int run_queue(int items, int n_valid, const std::vector<int>& order, std::vector<int>& per_xcd) {
    HostQueue q;
    std::vector<int> hits(n_valid > 0 ? n_valid : 1, 0);
    per_xcd.assign(8, 0);
    for (int b : order) {
        const int L = moe::xcd_queue_pick(b, n_valid, q);
        if (L >= n_valid || L < -1) {
            std::printf("queue: block %d -> %d outside [0, %d)\n", b, L, n_valid);
            return 1;
        }
        if (L >= 0) {
            ++hits[L];
            ++per_xcd[b % 8];
        }
    }
    for (int L = 0; L < n_valid; ++L)
        if (hits[L] != 1) {
            std::printf("queue: items %d n_valid %d: tile %d taken %d times\n", items, n_valid, L, hits[L]);
            return 1;
        }
    return 0;
}

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
    // the work queues: blocks in launch order, one XCD's blocks all before the
    // next XCD's (the first XCD fastest), and shuffled
    std::mt19937 rng(7);
    int max_gain = 0;
    for (int items = 0; items <= 2600; items += (items < 700 ? 1 : 13)) {
        const int grid = (int)moe::xcd_queue_grid(items);
        if (grid % 8 || grid < items || (items == 0) != (grid == 0)) {
            std::printf("bad queue grid %d for %d items\n", grid, items);
            return 1;
        }
        for (int n_valid = 0; n_valid <= items; n_valid += (n_valid < 300 ? 1 : 11)) {
            // every XCD holds its static blocks and a tail's worth more
            if (moe::xcd_queue_static(n_valid) > 0 && grid / 8 < moe::xcd_queue_static(n_valid) + moe::kQueueTail) {
                std::printf("queue grid %d too small for %d tiles\n", grid, n_valid);
                return 1;
            }
            std::vector<int> order(grid), per_xcd;
            for (int b = 0; b < grid; ++b) order[b] = b;
            if (run_queue(items, n_valid, order, per_xcd)) return 1;
            std::vector<int> by_xcd;
            for (int x = 0; x < 8; ++x)
                for (int b = x; b < grid; b += 8) by_xcd.push_back(b);
            if (run_queue(items, n_valid, by_xcd, per_xcd)) return 1;
            const int gain = per_xcd[0] - moe::xcd_share(0, n_valid);
            if (gain < 0 || (n_valid >= 8 * (moe::kQueueTail + 1) && gain < moe::kQueueTail)) {
                std::printf("queue: items %d n_valid %d: the first XCD took %d tiles over its share\n", items,
                            n_valid, gain);
                return 1;
            }
            max_gain = std::max(max_gain, gain);
            std::shuffle(order.begin(), order.end(), rng);
            if (run_queue(items, n_valid, order, per_xcd)) return 1;
            ++checked;
        }
    }
    std::printf("queue: a fast XCD took up to %d tiles over its share\n", max_gain);
    // the case of a grid that is not a multiple of 8 leaves tiles out (the
    // reason for xcd_grid): 46 blocks, 42 valid tiles
    int hit41 = 0;
    for (int b = 0; b < 46; ++b) hit41 += moe::xcd_remap(b, 42) == 41;
    std::printf("checked %ld (items, n_valid) pairs; unrounded grid 46 reaches tile 41: %d\n", checked, hit41);
    return hit41 == 0 ? 0 : 2;
}
