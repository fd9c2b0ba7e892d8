// workspace.hpp -- layout of the caller-owned device workspace.
//
//   [0,   128)  moegg_stats_t (device-written padding accounting)
//   [128, 256)  control block: tile count, chosen block_m, candidate tile counts
//   [256, ...)  int64 offsets[G + 1]  (segment starts / K-grouped row offsets)
//   [...]       int32 order[G]        (K-grouped: experts, longest first)
//   [...]       int64 groups[G + 1]   (K-grouped fp8: first 128-row scale group of each expert)
//   [...]       moegg_tile_t tiles[max_tiles]
//   [...]       uint32 sync[max_tiles]        (fused expert MLP: per-row-tile completion counters)
// Every region starts on a 256-byte boundary.  The regions up to `tiles` depend
// on G alone; `sync` follows the tile list, so its offset also depends on max_rows.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/moegg.h"

namespace moegg {

constexpr int kMaxExperts = 4096;
constexpr int kMinBlockM = 64;     // smallest schedulable tile height
constexpr int kExecRows = 16;      // MFMA row block: rows are executed in 16s
constexpr int kNumCand = 3;        // candidate tile heights 64, 128, 256

// Tag of a valid exemplar-selector state in the control block.
constexpr uint64_t kSelectorTag = 0x4D4F454753454C31ull;

struct Control {
    int32_t n_tiles;               // entries in the tile list
    int32_t block_m;               // tile height used
    int32_t cand_tiles[kNumCand];  // tiles(q) for q = 64, 128, 256
    int32_t G;                     // expert count of the last scheduled call
    // exemplar selector: the exemplar the last moegg_schedule_exemplar call on
    // this workspace chose (valid when sel_tag == kSelectorTag), and the
    // descriptor and distance of that call's histogram
    uint64_t sel_tag;
    int32_t sel_prev;
    int32_t sel_size_class;
    int32_t sel_lorenz[8];
    int64_t sel_distance;
    int32_t pad[12];
};
static_assert(sizeof(moegg_stats_t) <= 128, "stats block");
static_assert(sizeof(Control) == 128, "control block");

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
    size_t stats, control, offsets, order, groups, tiles, sync, total;
    int64_t max_tiles;
};

__host__ __device__ inline WsLayout ws_layout(int G, int64_t max_rows) {
    WsLayout L;
    L.stats = 0;
    L.control = 128;
    L.offsets = 256;
    L.order = L.offsets + align256(sizeof(int64_t) * (size_t)(G + 1));
    L.groups = L.order + align256(sizeof(int32_t) * (size_t)G);
    L.tiles = L.groups + align256(sizeof(int64_t) * (size_t)(G + 1));
    L.max_tiles = (max_rows + kMinBlockM - 1) / kMinBlockM + G;
    L.sync = L.tiles + align256(sizeof(moegg_tile_t) * (size_t)L.max_tiles);
    L.total = L.sync + align256(sizeof(uint32_t) * (size_t)L.max_tiles);
    return L;
}

}  // namespace moegg
