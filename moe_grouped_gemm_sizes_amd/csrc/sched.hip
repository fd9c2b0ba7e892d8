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

constexpr int kSchedThreads = 256;                          // 4 waves
constexpr int kWaves = kSchedThreads / 64;

__device__ __forceinline__ int64_t align_up64(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Block-wide exclusive scan of one int64 per thread: wave shuffles, then the
// four wave totals through LDS.  Two barriers.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* wave_buf, int64_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int64_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wave_buf[wave] = incl;
    __syncthreads();
    int64_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int64_t x = wave_buf[w];
        if (w < wave) base += x;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// Block-wide sums of NV int64 values per thread, all at once: two barriers.
template <int NV>
__device__ void block_sums(int64_t (&v)[NV], int64_t (*wave_buf)[NV]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v[i] += __shfl_xor(v[i], off, 64);
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < NV; ++i) wave_buf[wave][i] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int64_t t = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t += wave_buf[w][i];
        v[i] = t;
    }
    __syncthreads();
}

// Tile-height cost over the candidates 64, 128, 256 and per-expert heights.
// A launch holds one 512-thread tile per CU (256 CUs).  Each "wave" of 256
// tiles costs its tile height in rows plus a fixed per-tile overhead, so
//     cost(q) = ceil(tiles(q) * n_col_tiles / 256) * (q + 64).
// Per-expert heights run three classes of tiles (256-row tiles, remainders of
// 65..128 rows on 128-row tiles, remainders of 1..64 rows on 64-row tiles);
// each class is costed as its own sequence of waves:
//     cost_pe = sum over classes c of ceil(n_c * n_col_tiles / 256) * (q_c + 64).
// Ties go to the larger uniform q, which reuses weights better, and a uniform
// height wins a tie with per-expert heights.
__device__ int choose_block_m(const int64_t* cand_tiles, int64_t n_tail128, int64_t n_tail64, int n_col_tiles) {
    const int qs[kNumCand] = {64, 128, 256};
    auto waves = [&](int64_t tiles, int q) { return (tiles * n_col_tiles + 255) / 256 * (int64_t)(q + 64); };
    int best = 256;
    int64_t best_cost = -1;
    for (int c = kNumCand - 1; c >= 0; --c) {
        const int64_t cost = waves(cand_tiles[c], qs[c]);
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = qs[c]; }
    }
    const int64_t cost_pe =
        waves(cand_tiles[kNumCand - 1] - n_tail128 - n_tail64, 256) + waves(n_tail128, 128) + waves(n_tail64, 64);
    return cost_pe < best_cost ? MOEGG_BLOCK_M_PER_EXPERT : best;
}

// Quarter-octave size class of U: 4 * floor(log2 U) plus the two bits below
// U's leading one; 0 for U = 0.
__device__ __forceinline__ int32_t size_class(int64_t U) {
    if (U <= 0) return 0;
    const int e = 63 - __builtin_clzll((unsigned long long)U);
    const int64_t frac = e >= 2 ? (U >> (e - 2)) & 3 : (U << (2 - e)) & 3;
    return 4 * e + (int32_t)frac;
}

__device__ __forceinline__ bool valid_block_m_dev(int b) {
    return b == 64 || b == 128 || b == 256 || b == MOEGG_BLOCK_M_PER_EXPERT;
}

// Distribution-aware choice ("Adapt kernels without adding a CPU stall" on the
// MoE GroupGEMM padding page): sort the counts, normalize their top-k sums by
// U into an eight-point concentration curve, and take the nearest exemplar,
// keeping the workspace's previous exemplar while it is within `hysteresis`
// of the nearest.  Called by all threads after the accounting; the counts
// are in m_s.  Each thread scores its own exemplars (at most 256, so one
// each), so the table is read once, in parallel.  Returns the exemplar's
// block_m (or -2 when it names no valid one).  Thread 0 records the
// selection in the control block.
__device__ int select_exemplar(const int32_t* m_s, int32_t* srt_s, int64_t (*lor_buf)[8], int64_t* dist_s, int G,
                               int64_t U, const moegg_exemplar_t* __restrict__ ex, int n_ex, int hysteresis,
                               Control* ctl, int* bm_s) {
    const int t = threadIdx.x;
    // 1. bitonic sort, descending, over the next power of two (padded with zeros)
    int P = 1;
    while (P < G) P <<= 1;
    for (int i = t; i < P; i += kSchedThreads) srt_s[i] = i < G ? m_s[i] : 0;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = t; i < P; i += kSchedThreads) {
                const int l = i ^ j;
                if (l > i) {
                    const int32_t a = srt_s[i], b = srt_s[l];
                    const bool down = (i & k) == 0;
                    if (down ? a < b : a > b) { srt_s[i] = b; srt_s[l] = a; }
                }
            }
            __syncthreads();
        }
    }
    // 2. sums of the k_q = ceil(G (q + 1) / 8) largest counts
    int64_t top[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) top[q] = 0;
    for (int i = t; i < G; i += kSchedThreads) {
        const int64_t m = srt_s[i];
#pragma unroll
        for (int q = 0; q < 8; ++q) top[q] += i < (G * (q + 1) + 7) / 8 ? m : 0;
    }
    block_sums<8>(top, lor_buf);               // every thread now holds the eight sums
    // 3. descriptor (every thread), one exemplar's distance per thread into LDS
    int32_t lor[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) lor[q] = U > 0 ? (int32_t)((top[q] << 16) / U) : 0;
    const int32_t sc = size_class(U);
    for (int x = t; x < n_ex; x += kSchedThreads) {
        int64_t d = (int64_t)MOEGG_EXEMPLAR_SIZE_WEIGHT * llabs((int64_t)sc - ex[x].size_class);
#pragma unroll
        for (int q = 0; q < 8; ++q) d += llabs((int64_t)lor[q] - ex[x].lorenz[q]);
        dist_s[x] = d;
    }
    __syncthreads();
    // 4. nearest exemplar, ties to the lower index: wave 0 scans, then a shuffle
    //    reduction over (distance, index); thread 0 applies the hysteresis
    if (t < 64) {
        int64_t best_d = INT64_MAX;
        int best = n_ex;
        for (int x = t; x < n_ex; x += 64)
            if (dist_s[x] < best_d) { best_d = dist_s[x]; best = x; }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const int64_t od = __shfl_xor(best_d, off, 64);
            const int ob = __shfl_xor(best, off, 64);
            if (od < best_d || (od == best_d && ob < best)) { best_d = od; best = ob; }
        }
        if (t == 0) {
            int chosen = best;
            int64_t chosen_d = best_d;
            if (ctl->sel_tag == kSelectorTag && ctl->sel_prev >= 0 && ctl->sel_prev < n_ex) {
                const int64_t dp = dist_s[ctl->sel_prev];
                if (dp <= best_d + hysteresis) { chosen = ctl->sel_prev; chosen_d = dp; }
            }
            const int bm = ex[chosen].block_m;
            *bm_s = valid_block_m_dev(bm) ? bm : -2;
            ctl->sel_tag = kSelectorTag;
            ctl->sel_prev = chosen;
            ctl->sel_size_class = sc;
#pragma unroll
            for (int q = 0; q < 8; ++q) ctl->sel_lorenz[q] = lor[q];
            ctl->sel_distance = chosen_d;
        }
    }
    __syncthreads();
    return *bm_s;
}

// mode 0: contiguous layout (segment starts from aligned counts, tile list).
// mode 1: masked layout (segment starts e * cap, counts clamped to cap,
//         stats only: the masked kernel reads masked_m itself).
// Thread t owns a contiguous run of ceil(G / 256) experts, so block scans run
// in expert order and, up to 256 experts, every per-expert loop runs once.
// Those loops stay rolled (values go through LDS) to keep the kernel's code
// small: it runs cold before every GEMM.  It also zeroes n_clear words at
// clear (the expert MLP's completion counters), so a captured call needs no
// memset node.
__global__ __launch_bounds__(kSchedThreads) void sched_kernel(
    const int32_t* __restrict__ counts, int G, int64_t rows_total, int seg_align, int cap,
    int mode, int block_m_req, int n_col_tiles, int exec_block_m, unsigned char* __restrict__ ws,
    int64_t max_tiles, const moegg_exemplar_t* __restrict__ exemplars, int n_ex, int hysteresis,
    uint32_t* __restrict__ clear, int64_t n_clear) {
    for (int64_t i = threadIdx.x; i < n_clear; i += kSchedThreads) clear[i] = 0u;   // a caller's counters
    constexpr int NV = 3 + MOEGG_NUM_Q + kNumCand + 2;       // U, active, sum_sq, P(q) x6, tiles(q) x3, tails x2
    __shared__ int64_t wave_buf[kWaves];
    __shared__ int64_t sums_buf[kWaves][NV];
    __shared__ int32_t m_s[kMaxExperts];                     // clamped (then truncated) counts
    __shared__ int64_t start_s[kMaxExperts];                 // segment starts
    __shared__ unsigned int flags_s;
    __shared__ int32_t toff_s[kMaxExperts + 1];             // first tile of each expert
    __shared__ int32_t srt_s[kMaxExperts];                   // exemplar mode: sorted counts
    __shared__ int64_t lor_buf[kWaves][8];
    __shared__ int64_t dist_s[MOEGG_MAX_EXEMPLARS];           // exemplar mode: distances
    __shared__ int bm_s;
    const int t = threadIdx.x;
    const int ept = (G + kSchedThreads - 1) / kSchedThreads;  // experts per thread, contiguous
    const int e0 = min(G, t * ept), e1 = min(G, e0 + ept);
    WsLayout L = ws_layout(G, 0);
    moegg_stats_t* st = (moegg_stats_t*)(ws + L.stats);
    Control* ctl = (Control*)(ws + L.control);
    int64_t* offsets = (int64_t*)(ws + L.offsets);
    moegg_tile_t* tiles = (moegg_tile_t*)(ws + L.tiles);
    if (t == 0) flags_s = 0;

    // 1. count intake, clamped; segment sizes in the layout
    unsigned int flags = 0;
    int64_t seg_local = 0;
#pragma unroll 1
    for (int e = e0; e < e1; ++e) {
        int32_t m = counts[e];
        if (m < 0) { m = 0; flags |= MOEGG_FLAG_NEGATIVE_COUNT; }
        if (mode == 1 && m > cap) { m = cap; flags |= MOEGG_FLAG_COUNT_OVER_CAP; }
        m_s[e] = m;
        seg_local += mode == 1 ? cap : (m + seg_align - 1) / seg_align * seg_align;
    }
    // 2. prefix sums of segment sizes -> segment starts; truncate at rows_total
    int64_t seg_total;
    int64_t base = block_exclusive_scan(seg_local, wave_buf, &seg_total);
#pragma unroll 1
    for (int e = e0; e < e1; ++e) {
        const int32_t m = m_s[e];
        const int64_t seg = mode == 1 ? cap : (m + seg_align - 1) / seg_align * seg_align;
        int64_t room = rows_total - base;
        if (room < 0) room = 0;
        if ((int64_t)m > room) { m_s[e] = (int32_t)room; flags |= MOEGG_FLAG_ROWS_OVERFLOW; }
        start_s[e] = base;
        offsets[e] = base;
        base += seg;
    }
    if (t == 0) offsets[G] = seg_total;

    // 3. exact accounting, one fused block reduction (tile heights are powers of two)
    int64_t v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = 0;
#pragma unroll 1
    for (int e = e0; e < e1; ++e) {
        const int64_t m = m_s[e];
        v[0] += m;
        v[1] += m > 0;
        v[2] += m * m;
#pragma unroll
        for (int i = 0; i < MOEGG_NUM_Q; ++i) v[3 + i] += ((m + (8 << i) - 1) >> (3 + i)) << (3 + i);
#pragma unroll
        for (int c = 0; c < kNumCand; ++c) v[3 + MOEGG_NUM_Q + c] += (m + (64 << c) - 1) >> (6 + c);
        // rows of the last 256-row tile, 1..256: per-expert remainder classes
        const int64_t r = m - (((m + 255) >> 8) - 1) * 256;
        v[3 + MOEGG_NUM_Q + kNumCand] += m > 0 && r > 64 && r <= 128;
        v[3 + MOEGG_NUM_Q + kNumCand + 1] += m > 0 && r <= 64;
    }
    if (flags) atomicOr(&flags_s, flags);
    block_sums<NV>(v, sums_buf);       // its barriers also publish m_s, start_s and flags_s

    // 4. tile height (per-expert mode lists 256-row tiles): requested, matched
    //    to an exemplar, or from the cost rule
    int bm = block_m_req;
    if (mode == 1) {
        bm = exec_block_m;
    } else if (n_ex > 0) {
        bm = select_exemplar(m_s, srt_s, lor_buf, dist_s, G, v[0], exemplars, n_ex, hysteresis, ctl, &bm_s);
        if (bm == -2) {
            bm = 0;
            if (t == 0) flags_s |= MOEGG_FLAG_BAD_EXEMPLAR;
        }
    }
    if (mode == 0 && bm == 0)
        bm = choose_block_m(&v[3 + MOEGG_NUM_Q], v[3 + MOEGG_NUM_Q + kNumCand], v[3 + MOEGG_NUM_Q + kNumCand + 1],
                            n_col_tiles);
    const bool per_expert = bm == MOEGG_BLOCK_M_PER_EXPERT;
    const int bmt = per_expert ? 256 : bm;
    const int lg = 31 - __builtin_clz(bmt);                 // a power of two

    // 5. tile list (contiguous mode): expert ascending, tile ascending.  Each
    //    expert's first tile index goes to LDS; then every thread writes tiles
    //    t, t + 256, ... and finds each tile's expert by binary search.
    //    Per-expert mode: the tiles holding more than 128 valid rows come first
    //    (expert, tile ascending); then each expert's remainder tile of 65..128
    //    rows, then of 1..64 rows, in expert order.  Class of expert e's last
    //    tile: 0 (> 128 rows), 1 (65..128), 2 (1..64).
    auto tail_class = [&](int m) -> int {
        if (!per_expert || m <= 0) return 0;
        const int r = m - (((m + 255) >> 8) - 1) * 256;      // rows of the last tile, 1..256
        return r > 128 ? 0 : (r > 64 ? 1 : 2);
    };
    int64_t my_tiles = 0, my_tails = 0;                      // tails: class-1 count | class-2 count << 32
#pragma unroll 1
    for (int e = e0; e < e1; ++e) {
        const int c = tail_class(m_s[e]);
        my_tiles += ((m_s[e] + bmt - 1) >> lg) - (c ? 1 : 0);
        my_tails += c == 1 ? 1 : (c == 2 ? (int64_t)1 << 32 : 0);
    }
    int64_t n_main, n_tails;
    int64_t tbase = block_exclusive_scan(my_tiles, wave_buf, &n_main);
    int64_t tails_base = block_exclusive_scan(my_tails, wave_buf, &n_tails);
    const int64_t n1 = n_tails & 0xffffffff, n2 = n_tails >> 32;
    const int64_t n_tiles = n_main + n1 + n2;
    if (mode == 0) {
        int64_t b1 = n_main + (tails_base & 0xffffffff), b2 = n_main + n1 + (tails_base >> 32);
#pragma unroll 1
        for (int e = e0; e < e1; ++e) {
            const int m = m_s[e];
            const int c = tail_class(m);
            toff_s[e] = (int32_t)tbase;
            tbase += ((m + bmt - 1) >> lg) - (c ? 1 : 0);
            if (c) {
                const int i = ((m + 255) >> 8) - 1;
                const int64_t slot = c == 1 ? b1++ : b2++;
                if (slot < max_tiles) {
                    moegg_tile_t tl;
                    tl.expert = e;
                    tl.tile = i;
                    tl.row_start = (int32_t)(start_s[e] + (int64_t)i * 256);
                    tl.rows_valid = m - i * 256;
                    tiles[slot] = tl;
                }
            }
        }
        if (t == 0) toff_s[G] = (int32_t)n_main;
        __syncthreads();
        const int nt_all = (int)(n_main < max_tiles ? n_main : max_tiles);
#pragma unroll 1
        for (int T = t; T < nt_all; T += kSchedThreads) {
            int lo = 0, hi = G - 1;                          // last e with toff_s[e] <= T
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (toff_s[mid] <= T) lo = mid;
                else hi = mid - 1;
            }
            const int i = T - toff_s[lo];
            moegg_tile_t tl;
            tl.expert = lo;
            tl.tile = i;
            tl.row_start = (int32_t)(start_s[lo] + ((int64_t)i << lg));
            tl.rows_valid = min(bmt, m_s[lo] - (i << lg));
            tiles[T] = tl;
        }
    }

    // 6. stats and control block
    if (t == 0) {
        const int64_t layout_rows = mode == 1 ? (int64_t)G * cap : rows_total;
        st->U = v[0];
        st->P_exec = v[3 + 1];   // tiles skip whole 16-row MFMA blocks past their valid rows
        st->tiles = n_tiles;
        st->active = v[1];
        st->sum_sq = v[2];
        st->capacity_rows = layout_rows - v[0];
        for (int i = 0; i < MOEGG_NUM_Q; ++i) st->P_at[i] = v[3 + i];
        st->block_m = bm;
        st->error_flags = flags_s | (n_tiles > max_tiles ? MOEGG_FLAG_ROWS_OVERFLOW : 0u);
        ctl->n_tiles = (int32_t)(n_tiles < max_tiles ? n_tiles : max_tiles);
        ctl->block_m = bm;
        ctl->G = G;
        for (int c = 0; c < kNumCand; ++c) ctl->cand_tiles[c] = (int32_t)v[3 + MOEGG_NUM_Q + c];
    }
}

// K-grouped weight gradient: row offsets of each expert's segment along the
// reduction axis, the first 128-row scale group of each segment (fp8 operands:
// groups restart at every segment start), and the expert order for launch
// (longest first, ties by expert index).  The order comes from a bitonic sort
// of 64-bit keys (count << 32 | (4095 - expert)) in LDS, descending.
// scale_groups: rows of the fp8 scale arrays (0 for bf16); a histogram needing
// more groups than that sets MOEGG_FLAG_SCALE_GROUPS.
__global__ __launch_bounds__(kSchedThreads) void sched_k_grouped_kernel(
    const int32_t* __restrict__ t_sizes, int G, int64_t T, int64_t scale_groups, unsigned char* __restrict__ ws) {
    __shared__ int64_t wave_buf[kWaves];
    __shared__ int64_t sums_buf[kWaves][3];
    __shared__ int64_t key_s[kMaxExperts];
    __shared__ unsigned int flags_s;
    const int t = threadIdx.x;
    WsLayout L = ws_layout(G, 0);
    moegg_stats_t* st = (moegg_stats_t*)(ws + L.stats);
    Control* ctl = (Control*)(ws + L.control);
    int64_t* offsets = (int64_t*)(ws + L.offsets);
    int64_t* groups = (int64_t*)(ws + L.groups);
    int32_t* order = (int32_t*)(ws + L.order);
    if (t == 0) flags_s = 0;
    unsigned int flags = 0;
    const int ept = (G + kSchedThreads - 1) / kSchedThreads;
    const int e0 = min(G, t * ept), e1 = min(G, e0 + ept);
    int64_t local = 0;
#pragma unroll 1
    for (int e = e0; e < e1; ++e) {
        int32_t m = t_sizes[e];
        if (m < 0) { m = 0; flags |= MOEGG_FLAG_NEGATIVE_COUNT; }
        key_s[e] = m;
        local += m;
    }
    int64_t tot;
    int64_t base = block_exclusive_scan(local, wave_buf, &tot);
    // segments truncated at T: the counts that are actually used, then their groups
    int64_t v[3] = {0, 0, 0};
    int64_t grp_local = 0;
#pragma unroll 1
    for (int e = e0; e < e1; ++e) {
        const int64_t m_in = key_s[e];
        int64_t m = m_in;
        int64_t room = T - base;
        if (room < 0) room = 0;
        if (m > room) { m = room; flags |= MOEGG_FLAG_ROWS_OVERFLOW; }
        offsets[e] = base;
        key_s[e] = m;
        v[0] += m;
        v[1] += m > 0;
        v[2] += m * m;
        grp_local += (m + 127) / 128;
        base += m_in;
    }
    int64_t grp_tot;
    int64_t gbase = block_exclusive_scan(grp_local, wave_buf, &grp_tot);   // barriers publish key_s too
#pragma unroll 1
    for (int e = e0; e < e1; ++e) {
        groups[e] = gbase;
        gbase += (key_s[e] + 127) / 128;
    }
    // offsets[e] are the layout's segment starts; segments truncated at T end there
    if (t == 0) {
        offsets[G] = tot < T ? tot : T;
        groups[G] = grp_tot;
    }
    if (scale_groups > 0 && grp_tot > scale_groups) flags |= MOEGG_FLAG_SCALE_GROUPS;
    if (flags) atomicOr(&flags_s, flags);
    block_sums<3>(v, sums_buf);        // its barriers also publish flags_s
    // longest first: sort keys descending over the next power of two (padding -1 sorts last)
    int P = 1;
    while (P < G) P <<= 1;
    for (int e = t; e < P; e += kSchedThreads)
        key_s[e] = e < G ? (key_s[e] << 32) | (int64_t)(kMaxExperts - 1 - e) : -1;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = t; i < P; i += kSchedThreads) {
                const int l = i ^ j;
                if (l > i) {
                    const int64_t a = key_s[i], b = key_s[l];
                    const bool down = (i & k) == 0;
                    if (down ? a < b : a > b) { key_s[i] = b; key_s[l] = a; }
                }
            }
            __syncthreads();
        }
    }
    for (int r = t; r < G; r += kSchedThreads) order[r] = kMaxExperts - 1 - (int32_t)(key_s[r] & 0xFFFFFFFF);
    if (t == 0) {
        st->U = v[0];
        st->P_exec = v[0];
        st->tiles = 0;
        st->active = v[1];
        st->sum_sq = v[2];
        st->capacity_rows = T - v[0];
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
                        hipStream_t stream, uint32_t* clear, int64_t n_clear) {
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, stream, counts, G, rows_total, seg_align,
                       cap, mode, block_m_req, n_col_tiles, exec_block_m, (unsigned char*)ws, max_tiles,
                       (const moegg_exemplar_t*)nullptr, 0, 0, clear, n_clear);
    return hipGetLastError();
}

hipError_t launch_sched_exemplar(const int32_t* counts, int G, int64_t rows_total, int seg_align, int n_col_tiles,
                                 const moegg_exemplar_t* exemplars, int n_ex, int hysteresis, void* ws,
                                 int64_t max_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, stream, counts, G, rows_total, seg_align, 0,
                       0, 0, n_col_tiles, 0, (unsigned char*)ws, max_tiles, exemplars, n_ex, hysteresis,
                       (uint32_t*)nullptr, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_sched_k_grouped(const int32_t* t_sizes, int G, int64_t T, int64_t scale_groups, void* ws,
                                  hipStream_t stream) {
    hipLaunchKernelGGL(sched_k_grouped_kernel, dim3(1), dim3(kSchedThreads), 0, stream, t_sizes, G, T,
                       scale_groups, (unsigned char*)ws);
    return hipGetLastError();
}

}  // namespace moegg
