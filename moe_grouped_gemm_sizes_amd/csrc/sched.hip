// sched.hip -- device-side scheduler: per-expert counts -> padding accounting,
// tile height choice and the flat tile work list, in one workgroup, with no
// host round trip.
//
// It follows these passages:
//   - "MoE GroupGEMM padding under expert skew", section "Calculate padded
//     token columns": U = sum m_e; P(q) = sum over active experts of
//     q * ceil(m_e / q), where an inactive expert adds nothing.
//   - Same page, section "Summarize skew without losing the histogram": the
//     sum of squares behind effective experts.
//   - Same page, section "Grouped execution does not require padded experts":
//     the work list is built from each expert's actual count.  Zero-sized
//     experts get no tiles, so their weights are never loaded.  The last tile
//     of an expert carries only its remaining rows.
//   - Same page, section "Adapt kernels without adding a CPU stall": the
//     histogram stays on the GPU, and the tile height is chosen there.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"
#include "workspace.hpp"

namespace moegg {

constexpr int kSchedThreads = 1024;
constexpr int kPerThread = kMaxExperts / kSchedThreads;   // 4 experts per thread
static_assert(kPerThread * kSchedThreads == kMaxExperts, "sched sizing");

__device__ __forceinline__ int64_t align_up64(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Block-wide exclusive scan of one int64 value per thread (1024 threads).
// Returns the exclusive prefix and writes the block total to *total.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* buf, int64_t* total) {
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
        int64_t add = t >= off ? buf[t - off] : 0;
        __syncthreads();
        buf[t] += add;
        __syncthreads();
    }
    int64_t incl = buf[t];
    *total = buf[kSchedThreads - 1];
    __syncthreads();
    return incl - v;
}

__device__ int64_t block_sum(int64_t v, int64_t* buf) {
    int64_t tot;
    block_exclusive_scan(v, buf, &tot);
    return tot;
}

// Tile-height cost over the candidates 64, 128, 256.  A launch holds one
// 512-thread tile per CU (256 CUs).  Each "wave" of 256 tiles costs its tile
// height in rows plus a fixed per-tile overhead, so
//     cost(q) = ceil(tiles(q) * n_col_tiles / 256) * (q + 64).
// Ties go to the larger q, which reuses weights better.
__device__ int choose_block_m(const int32_t* cand_tiles, int n_col_tiles) {
    const int qs[kNumCand] = {64, 128, 256};
    int best = 256;
    int64_t best_cost = -1;
    for (int c = kNumCand - 1; c >= 0; --c) {
        int64_t items = (int64_t)cand_tiles[c] * n_col_tiles;
        int64_t cost = (items + 255) / 256 * (int64_t)(qs[c] + 64);
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = qs[c]; }
    }
    return best;
}

// mode 0: contiguous layout (segment starts from aligned counts, tile list).
// mode 1: masked layout (segment starts e * cap, counts clamped to cap,
//         stats only: the masked kernel reads masked_m itself).
__global__ __launch_bounds__(kSchedThreads) void sched_kernel(
    const int32_t* __restrict__ counts, int G, int64_t rows_total, int seg_align, int cap,
    int mode, int block_m_req, int n_col_tiles, int exec_block_m, unsigned char* __restrict__ ws,
    int64_t max_tiles) {
    __shared__ int64_t scan_buf[kSchedThreads];
    __shared__ int64_t seg_off_s[kMaxExperts];
    __shared__ int32_t m_s[kMaxExperts];
    __shared__ int32_t chosen_s;
    __shared__ uint32_t flags_s;
    const int t = threadIdx.x;
    WsLayout L = ws_layout(G, 0);
    moegg_stats_t* st = (moegg_stats_t*)(ws + L.stats);
    Control* ctl = (Control*)(ws + L.control);
    int64_t* offsets = (int64_t*)(ws + L.offsets);
    moegg_tile_t* tiles = (moegg_tile_t*)(ws + L.tiles);

    if (t == 0) flags_s = 0;
    __syncthreads();

    // 1. count intake, clamped; segment sizes in the layout
    uint32_t flags = 0;
    int64_t seg_local = 0;
    int32_t m_loc[kPerThread];
    int64_t seg_loc[kPerThread];
    for (int j = 0; j < kPerThread; ++j) {
        int e = t * kPerThread + j;
        int32_t m = 0;
        if (e < G) {
            m = counts[e];
            if (m < 0) { m = 0; flags |= MOEGG_FLAG_NEGATIVE_COUNT; }
            if (mode == 1 && m > cap) { m = cap; flags |= MOEGG_FLAG_COUNT_OVER_CAP; }
        }
        m_loc[j] = m;
        seg_loc[j] = e < G ? (mode == 1 ? (int64_t)cap : align_up64(m, seg_align)) : 0;
        seg_local += seg_loc[j];
    }
    // 2. prefix sums of segment sizes -> segment starts
    int64_t seg_total;
    int64_t base = block_exclusive_scan(seg_local, scan_buf, &seg_total);
    for (int j = 0; j < kPerThread; ++j) {
        int e = t * kPerThread + j;
        if (e < G) {
            int64_t start = base;
            // truncate segments that run past the end of the buffer
            int64_t room = rows_total - start;
            if (room < 0) room = 0;
            if ((int64_t)m_loc[j] > room) { m_loc[j] = (int32_t)room; flags |= MOEGG_FLAG_ROWS_OVERFLOW; }
            seg_off_s[e] = start;
            m_s[e] = m_loc[j];
            offsets[e] = start;
        }
        base += seg_loc[j];
    }
    if (t == 0) offsets[G] = seg_total;
    if (flags) atomicOr(&flags_s, flags);
    __syncthreads();

    // 3. exact accounting
    const int qs_all[MOEGG_NUM_Q] = {8, 16, 32, 64, 128, 256};
    int64_t u = 0, act = 0, sq = 0, p_at[MOEGG_NUM_Q] = {0, 0, 0, 0, 0, 0};
    int64_t cand[kNumCand] = {0, 0, 0};
    for (int j = 0; j < kPerThread; ++j) {
        int64_t m = m_loc[j];
        u += m;
        act += m > 0;
        sq += m * m;
        for (int i = 0; i < MOEGG_NUM_Q; ++i) p_at[i] += m > 0 ? align_up64(m, qs_all[i]) : 0;
        for (int c = 0; c < kNumCand; ++c) cand[c] += (m + (64 << c) - 1) / (64 << c);
    }
    int64_t U = block_sum(u, scan_buf);
    int64_t ACT = block_sum(act, scan_buf);
    int64_t SQ = block_sum(sq, scan_buf);
    int64_t P[MOEGG_NUM_Q];
    for (int i = 0; i < MOEGG_NUM_Q; ++i) P[i] = block_sum(p_at[i], scan_buf);
    int64_t CT[kNumCand];
    for (int c = 0; c < kNumCand; ++c) CT[c] = block_sum(cand[c], scan_buf);

    // 4. tile height
    if (t == 0) {
        int32_t ct32[kNumCand];
        for (int c = 0; c < kNumCand; ++c) ct32[c] = (int32_t)CT[c];
        int bm = block_m_req;
        if (mode == 1) bm = exec_block_m;
        else if (bm == 0) bm = choose_block_m(ct32, n_col_tiles);
        chosen_s = bm;
    }
    __syncthreads();
    const int bm = chosen_s;

    // 5. tile list (contiguous mode): expert ascending, tile ascending
    int64_t my_tiles = 0;
    for (int j = 0; j < kPerThread; ++j) my_tiles += (m_loc[j] + bm - 1) / bm;
    int64_t n_tiles;
    int64_t tbase = block_exclusive_scan(my_tiles, scan_buf, &n_tiles);
    if (mode == 0) {
        for (int j = 0; j < kPerThread; ++j) {
            int e = t * kPerThread + j;
            int32_t m = m_loc[j];
            int nt = (m + bm - 1) / bm;
            for (int i = 0; i < nt && tbase + i < max_tiles; ++i) {
                moegg_tile_t tl;
                tl.expert = e;
                tl.tile = i;
                tl.row_start = (int32_t)(seg_off_s[e] + (int64_t)i * bm);
                tl.rows_valid = min(bm, m - i * bm);
                tiles[tbase + i] = tl;
            }
            tbase += nt;
        }
    }

    // 6. stats and control block
    if (t == 0) {
        int64_t layout_rows = mode == 1 ? (int64_t)G * cap : rows_total;
        st->U = U;
        st->P_exec = P[1];   // tiles skip whole 16-row MFMA blocks past their valid rows
        st->tiles = n_tiles;
        st->active = ACT;
        st->sum_sq = SQ;
        st->capacity_rows = layout_rows - U;
        for (int i = 0; i < MOEGG_NUM_Q; ++i) st->P_at[i] = P[i];
        st->block_m = bm;
        st->error_flags = flags_s | (n_tiles > max_tiles ? MOEGG_FLAG_ROWS_OVERFLOW : 0u);
        ctl->n_tiles = (int32_t)(n_tiles < max_tiles ? n_tiles : max_tiles);
        ctl->block_m = bm;
        ctl->G = G;
        for (int c = 0; c < kNumCand; ++c) ctl->cand_tiles[c] = (int32_t)CT[c];
    }
}

// K-grouped weight gradient: row offsets of each expert's segment along the
// reduction axis, and the expert order for launch (longest first, ties by
// expert index).
__global__ __launch_bounds__(kSchedThreads) void sched_k_grouped_kernel(
    const int32_t* __restrict__ t_sizes, int G, int64_t T, unsigned char* __restrict__ ws) {
    __shared__ int64_t scan_buf[kSchedThreads];
    __shared__ int32_t m_s[kMaxExperts];
    __shared__ uint32_t flags_s;
    const int t = threadIdx.x;
    WsLayout L = ws_layout(G, 0);
    moegg_stats_t* st = (moegg_stats_t*)(ws + L.stats);
    Control* ctl = (Control*)(ws + L.control);
    int64_t* offsets = (int64_t*)(ws + L.offsets);
    int32_t* order = (int32_t*)(ws + L.order);
    if (t == 0) flags_s = 0;
    __syncthreads();
    uint32_t flags = 0;
    int32_t m_loc[kPerThread], m_in[kPerThread];
    int64_t local = 0;
    for (int j = 0; j < kPerThread; ++j) {
        int e = t * kPerThread + j;
        int32_t m = e < G ? t_sizes[e] : 0;
        if (m < 0) { m = 0; flags |= MOEGG_FLAG_NEGATIVE_COUNT; }
        m_loc[j] = m_in[j] = m;
        local += m;
    }
    int64_t tot;
    int64_t base = block_exclusive_scan(local, scan_buf, &tot);
    int64_t u = 0, act = 0, sq = 0;
    for (int j = 0; j < kPerThread; ++j) {
        int e = t * kPerThread + j;
        if (e < G) {
            int64_t room = T - base;
            if (room < 0) room = 0;
            if ((int64_t)m_loc[j] > room) { m_loc[j] = (int32_t)room; flags |= MOEGG_FLAG_ROWS_OVERFLOW; }
            offsets[e] = base;
            m_s[e] = m_loc[j];
            u += m_loc[j];
            act += m_loc[j] > 0;
            sq += (int64_t)m_loc[j] * m_loc[j];
        }
        base += m_in[j];
    }
    if (flags) atomicOr(&flags_s, flags);
    __syncthreads();
    // offsets[e] holds starts computed from the unclamped-to-T running sum;
    // truncated segments end at T, so the end offset is min(sum, T).
    if (t == 0) offsets[G] = tot < T ? tot : T;
    int64_t U = block_sum(u, scan_buf);
    int64_t ACT = block_sum(act, scan_buf);
    int64_t SQ = block_sum(sq, scan_buf);
    // rank = number of experts that come before e in longest-first order
    for (int e = t; e < G; e += kSchedThreads) {
        int32_t me = m_s[e];
        int r = 0;
        for (int j = 0; j < G; ++j) {
            int32_t mj = m_s[j];
            r += (mj > me) || (mj == me && j < e);
        }
        order[r] = e;
    }
    if (t == 0) {
        st->U = U;
        st->P_exec = U;
        st->tiles = 0;
        st->active = ACT;
        st->sum_sq = SQ;
        st->capacity_rows = T - U;
        for (int i = 0; i < MOEGG_NUM_Q; ++i) st->P_at[i] = 0;
        st->block_m = 0;
        st->error_flags = flags_s;
        ctl->n_tiles = 0;
        ctl->block_m = 0;
        ctl->G = G;
    }
}

}  // namespace moegg

// ------------------------------------------------------------------ launchers

namespace moegg {

hipError_t launch_sched(const int32_t* counts, int G, int64_t rows_total, int seg_align, int cap, int mode,
                        int block_m_req, int n_col_tiles, int exec_block_m, void* ws, int64_t max_tiles,
                        hipStream_t stream) {
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, stream, counts, G, rows_total, seg_align,
                       cap, mode, block_m_req, n_col_tiles, exec_block_m, (unsigned char*)ws, max_tiles);
    return hipGetLastError();
}

hipError_t launch_sched_k_grouped(const int32_t* t_sizes, int G, int64_t T, void* ws, hipStream_t stream) {
    hipLaunchKernelGGL(sched_k_grouped_kernel, dim3(1), dim3(kSchedThreads), 0, stream, t_sizes, G, T,
                       (unsigned char*)ws);
    return hipGetLastError();
}

}  // namespace moegg
