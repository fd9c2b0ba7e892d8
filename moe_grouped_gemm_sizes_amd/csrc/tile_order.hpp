// Order of the contiguous GEMM's and the one-launch expert MLP's work items
// over the scheduler's tile list.  Host and device code: a host test checks on
// the CPU that every (row tile, column tile) pair is handed out exactly once.
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

// Block -> work item: XCD x (= b % 8, the dispatcher's round robin over the
// eight XCDs) takes items in runs of 32, so each run of 256 blocks is one
// permutation of 256 items.
__host__ __device__ inline int block_to_item(int b) {
    return (b >> 8) * 256 + (b & 7) * 32 + ((b & 255) >> 3);
}

// Grid of the one-launch expert MLP over a 256-row tile list of at most
// max_rt row tiles: first the SwiGLU-projection (L1) items, max_rt * c1 of
// them rounded up to whole runs of 256 blocks, then the down-projection (L2)
// items, max_rt * c2 rounded likewise.  Every L1 block has a lower index than
// every L2 block.
__host__ __device__ inline int64_t mlp_l1_blocks(int64_t max_rt, int c1) { return (max_rt * c1 + 255) / 256 * 256; }
__host__ __device__ inline int64_t mlp_blocks(int64_t max_rt, int c1, int c2) {
    return mlp_l1_blocks(max_rt, c1) + (max_rt * c2 + 255) / 256 * 256;
}

// Block b of that grid -> phase (1 = L1, 2 = L2), row tile rt and column
// tile ct of an n_rt-tile list, each phase in the contiguous GEMM's order;
// false for a block with no item.
__host__ __device__ inline bool mlp_block_item(int b, int l1_blocks, int n_rt, int c1, int c2,
                                               const moegg_tile_t* tiles, int& phase, int& rt, int& ct) {
    const bool l1 = b < l1_blocks;
    const int nc = l1 ? c1 : c2;
    const int item = block_to_item(l1 ? b : b - l1_blocks);
    if (item >= n_rt * nc) return false;
    phase = l1 ? 1 : 2;
    item_to_list_tiles(item, n_rt, nc, tiles, false, rt, ct);
    return true;
}

}  // namespace moegg
