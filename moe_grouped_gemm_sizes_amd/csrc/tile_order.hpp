// Order of the contiguous GEMM's work items over the scheduler's tile list.
// Host and device code: a host test checks on the CPU that every (row tile,
// column tile) pair is handed out exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moegg.h"

namespace moegg {

// Work item -> (row tile rt, column tile ct) over a tile list: items run group by group, a
// group being up to four consecutive row tiles of one expert (tile indices 4j .. 4j+3 of
// that expert; a per-expert list's tails, rows <= 128, are groups of one), column tile
// slowest within a group.  A group never spans two experts, whose tiles share no weights.
__host__ __device__ inline void item_to_list_tiles(int item, int n_rt, int n_ct, const moegg_tile_t* tiles,
                                                   bool per_expert, int& rt, int& ct) {
    const int T = item / n_ct;
    const moegg_tile_t tT = tiles[T];
    int first = T, gm = 1;
    if (!(per_expert && tT.rows_valid <= 128)) {
        first = T - (tT.tile & 3);
#pragma unroll
        for (int k = 1; k < 4; ++k) {
            if (first + k >= n_rt) break;
            const moegg_tile_t tk = tiles[first + k];
            if (tk.expert != tT.expert || (per_expert && tk.rows_valid <= 128)) break;
            gm = k + 1;
        }
    }
    const int r = item - first * n_ct;
    ct = r / gm;
    rt = first + (r - ct * gm);
}

}  // namespace moegg
