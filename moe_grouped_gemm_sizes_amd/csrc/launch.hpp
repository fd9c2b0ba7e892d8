// launch.hpp -- host-side launcher interface between the C ABI (api.hip) and
// the kernels (sched.hip, gemm.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moegg.h"

namespace moegg {

struct ContigArgs {
    const void* A;
    const void* A_scale;          // fp32 [rows, K/128] or [K/128, rows_total], or E8M0 bytes [K/128, rows_total]
    const void* B;
    const void* B_scale;          // fp32 or E8M0 bytes [G, K/128, N/128]
    void* C;
    const int32_t* counts;        // m_sizes, or masked_m for the masked layout
    const unsigned char* ws;      // scheduler output (contiguous layout)
    int G, K, N, cap;             // cap: masked layout only
    int rows_total;               // rows of A and C (masked layout: G * cap)
    void* C_scale;                // SwiGLU with e4m3 output: fp32 [rows_total, N / 256] scales, else NULL
    int a_scale_km;               // fp32 activation scales (and C_scale) stored [K/128, rows_total]
    int req_block_m;              // contiguous: height the caller asked for (0 = whatever the schedule chose)
    int b_panel;                  // weights stored in column panels of the kernel's tile width (see moegg.h)
};

// Expert MLP in one launch: l1 is the SwiGLU projection (C = H,
// C_scale = H_scale, N = 2I), l2 the down projection on H (A = H, K = I, N = N2).
struct MlpArgs {
    ContigArgs l1, l2;
    uint32_t* sync;               // per-row-tile completion counters [max_tiles], zero at launch
    int l1_blocks;                // blocks [0, l1_blocks) run L1 items, the rest L2 items
};

struct KGroupedArgs {
    const void* X;
    const void* dY;
    float* dW;
    const unsigned char* ws;
    int G, Mw, Nw;
    const void* X_scale;           // fp8: [scale_groups, Mw] fp32 or E8M0 bytes, else NULL
    const void* dY_scale;          // fp8: [scale_groups, Nw] fp32 or E8M0 bytes, else NULL
    int64_t scale_groups;          // rows of the fp8 scale arrays
};

// mode 0: contiguous (tile list); mode 1: masked (stats only).
hipError_t launch_sched(const int32_t* counts, int G, int64_t rows_total, int seg_align, int cap, int mode,
                        int block_m_req, int n_col_tiles, int exec_block_m, void* ws, int64_t max_tiles,
                        hipStream_t stream, uint32_t* clear = nullptr, int64_t n_clear = 0);
// exemplar-matching tile height (moegg_schedule_exemplar); exemplars: device
// array of n_ex entries
hipError_t launch_sched_exemplar(const int32_t* counts, int G, int64_t rows_total, int seg_align, int n_col_tiles,
                                 const moegg_exemplar_t* exemplars, int n_ex, int hysteresis, void* ws,
                                 int64_t max_tiles, hipStream_t stream);
// scale_groups: rows of the K-grouped fp8 scale arrays (0 for bf16)
hipError_t launch_sched_k_grouped(const int32_t* t_sizes, int G, int64_t T, int64_t scale_groups, void* ws,
                                  hipStream_t stream);
// w4: packed E2M1 weights [G, N, K/2] (needs fp8 activations, E8M0 scales, !b_kn)
hipError_t launch_contiguous(const ContigArgs& a, bool fp8, bool e8m0, bool w4, bool b_kn, int64_t rows_total,
                             int block_m, hipStream_t s);
// L1 GEMM with the SwiGLU epilogue: [G, N, K] weights whose N columns interleave
// gate and up in groups of 16; C receives [rows_total, N / 2] bf16, or e4m3 codes
// with fp32 1x128 scales in C_scale when that is set
// w4: fp8 activations with E8M0 scales and packed E2M1 weights [G, N, K/2]
hipError_t launch_contiguous_swiglu(const ContigArgs& a, bool fp8, bool w4, int64_t rows_total, int block_m,
                                    hipStream_t s);
hipError_t launch_masked(const ContigArgs& a, bool fp8, bool e8m0, bool w4, bool b_kn, hipStream_t s);
hipError_t launch_k_grouped(const KGroupedArgs& a, bool fp8, bool e8m0, hipStream_t s);
// n_words 32-bit zeros at p (a fill kernel: graph-capturable, no memset node)
// the fused expert MLP on fp8 operands (e4m3 A, W1, H, W2 with fp32 scales); one workgroup per
// work item, n_workgroups at least the items the schedule can produce
hipError_t launch_mlp_fused(const MlpArgs& a, int n_workgroups, hipStream_t s);
int masked_block_m();
int masked_block_n();

}  // namespace moegg
