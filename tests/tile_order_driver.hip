// Host check of the contiguous GEMM's work order (csrc/tile_order.hpp): for each
// tile list in the input file, every item maps to a (row tile, column tile) in
// range, every pair is handed out exactly once, and an item's row tile belongs to
// the expert of the tile at index item / n_ct (groups never span two experts).  Input: per case a line
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
        ++cases;
    }
    fclose(f);
    if (fails) printf("%d failures\n", fails);
    else printf("%d cases ok\n", cases);
    return fails ? 1 : 0;
}
