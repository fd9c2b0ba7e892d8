// Host check of the contiguous GEMM's work order (csrc/tile_order.hpp): for each
// tile list in the input file, every item maps to a (row tile, column tile) in
// range, every pair is handed out exactly once, and an item's row tile belongs to
// the expert of the tile at index item / n_ct (groups never span two experts).
// For the one-launch expert MLP's grid over the same list: every (phase, row
// tile, column tile) once, all L1 blocks before all L2 blocks.  Input: per case a line
// "n_ct per_expert n_rt", then n_rt lines "expert tile rows_valid".  Prints
// "ok" or the first failures.
#include <stdio.h>

#include <set>
#include <utility>
#include <vector>

#include "../moe_grouped_gemm_sizes_amd/csrc/tile_order.hpp"

int main(int argc, char** argv) {
    if (argc != 2) return 2;
    FILE* f = fopen(argv[1], "r");
    if (!f) return 2;
    int n_ct, per_expert, n_rt, cases = 0, fails = 0;
    while (fscanf(f, "%d %d %d", &n_ct, &per_expert, &n_rt) == 3) {
        std::vector<moegg_tile_t> tiles(n_rt);
        for (int i = 0; i < n_rt; ++i) {
            if (fscanf(f, "%d %d %d", &tiles[i].expert, &tiles[i].tile, &tiles[i].rows_valid) != 3) return 2;
            tiles[i].row_start = 0;
        }
        std::set<std::pair<int, int>> seen;
        for (int item = 0; item < n_rt * n_ct; ++item) {
            int rt = -1, ct = -1;
            moegg::item_to_list_tiles(item, n_rt, n_ct, tiles.data(), per_expert != 0, rt, ct);
            // the item's group holds the tile at index item / n_ct, and a group stays within one expert
            if (rt < 0 || rt >= n_rt || ct < 0 || ct >= n_ct || !seen.insert({rt, ct}).second ||
                tiles[rt].expert != tiles[item / n_ct].expert) {
                if (fails < 20) printf("case %d item %d -> (%d, %d)\n", cases, item, rt, ct);
                ++fails;
            }
        }
        // the one-launch expert MLP's grid over the same list, as L1 with c1 = n_ct column tiles and L2 with
        // c2 = 2 n_ct + 1, sized for a few row tiles more than the list holds: each (phase, rt, ct) once, every
        // L1 block before every L2 block, and each run of 256 blocks one permutation of its 256 items
        if (!per_expert) {
            const int c1 = n_ct, c2 = 2 * n_ct + 1;
            const int64_t max_rt = n_rt + 3;
            const int l1 = (int)moegg::mlp_l1_blocks(max_rt, c1);
            const int64_t nb = moegg::mlp_blocks(max_rt, c1, c2);
            std::set<std::pair<int, int>> s1, s2;
            std::set<int> items;
            int last_l1 = -1, first_l2 = -1;
            bool bad = l1 % 256 != 0 || nb % 256 != 0 || l1 < max_rt * c1 || nb - l1 < max_rt * c2;
            for (int b = 0; b < nb; ++b) {
                if (b % 256 == 0) items.clear();
                if (!items.insert(moegg::block_to_item(b)).second || moegg::block_to_item(b) / 256 != b / 256)
                    bad = true;
                int phase = 0, rt = -1, ct = -1;
                if (!moegg::mlp_block_item(b, l1, n_rt, c1, c2, tiles.data(), phase, rt, ct)) continue;
                const int nc = phase == 1 ? c1 : c2;
                if (rt < 0 || rt >= n_rt || ct < 0 || ct >= nc ||
                    !(phase == 1 ? s1 : s2).insert({rt, ct}).second)
                    bad = true;
                if (phase == 1) last_l1 = b;
                else if (first_l2 < 0) first_l2 = b;
            }
            if (bad || (int64_t)s1.size() != (int64_t)n_rt * c1 || (int64_t)s2.size() != (int64_t)n_rt * c2 ||
                (n_rt > 0 && !(last_l1 < first_l2))) {
                if (fails < 20) printf("case %d: expert MLP grid\n", cases);
                ++fails;
            }
        }
        ++cases;
    }
    fclose(f);
    if (fails) printf("%d failures\n", fails);
    else printf("%d cases ok\n", cases);
    return fails ? 1 : 0;
}
