// api.hip -- the C ABI declared in include/moegg.h: argument validation,
// workspace layout and kernel launches.  No call here allocates device
// memory or synchronizes, except the two *_read calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/moegg.h"
#include "launch.hpp"
#include "tile_order.hpp"
#include "workspace.hpp"


using namespace moegg;

namespace {

const int64_t kMaxBufferBytes = 0xFFFFFFF0ll;   // one buffer resource spans < 4 GiB

bool debug_on() {
    static int on = -1;
    if (on < 0) {
        const char* v = getenv("MOEGG_DEBUG");
        on = (v && v[0] == '1') ? 1 : 0;
    }
    return on == 1;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

moegg_status_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MOEGG_OK;
    if (debug_on()) fprintf(stderr, "moegg: %s failed: %s\n", what, hipGetErrorString(e));
    return MOEGG_ERR_HIP;
}

// Weight layouts: N-contiguous rows (plain or in column panels), and whether paneled.
bool layout_kn(moegg_b_layout_t l) { return l == MOEGG_B_KN || l == MOEGG_B_KN_PANEL; }
bool layout_panel(moegg_b_layout_t l) { return l == MOEGG_B_KN_PANEL || l == MOEGG_B_NK_PANEL; }

// Block scales stored as E8M0 exponent bytes.
bool e8m0_scales(moegg_dtype_t d) { return d == MOEGG_FP8_E4M3_E8M0 || d == MOEGG_FP8_E4M3_FP4_E2M1; }

// Scales stored [groups, rows] (E8M0 bytes, or fp32 with MOEGG_FP8_E4M3_SCALE_KM)
// are addressed with 32-bit buffer offsets across the whole array, so
// groups * rows elements must stay within 4 GiB.
bool transposed_scales_fit(moegg_dtype_t d, int64_t groups, int64_t rows) {
    const int64_t esz = d == MOEGG_FP8_E4M3_SCALE_KM ? 4 : e8m0_scales(d) ? 1 : 0;
    return groups * rows * esz <= (int64_t)UINT32_MAX;
}

// Shared checks for the contiguous and masked calls.
moegg_status_t check_common(const void* A, const void* A_scale, const void* B, const void* B_scale,
                            const void* C, int G, int K, int N, moegg_dtype_t dtype, moegg_b_layout_t b_layout,
                            int col_tile) {
    if (!A || !B || !C) return MOEGG_ERR_INVALID_ARG;
    if (G < 1 || G > kMaxExperts || K < 1 || N < 1) return MOEGG_ERR_INVALID_ARG;
    if (dtype != MOEGG_BF16 && dtype != MOEGG_FP8_E4M3 && dtype != MOEGG_FP8_E4M3_E8M0 &&
        dtype != MOEGG_FP8_E4M3_FP4_E2M1 && dtype != MOEGG_FP8_E4M3_SCALE_KM)
        return MOEGG_ERR_INVALID_ARG;
    if (b_layout != MOEGG_B_KN && b_layout != MOEGG_B_NK && b_layout != MOEGG_B_KN_PANEL &&
        b_layout != MOEGG_B_NK_PANEL)
        return MOEGG_ERR_INVALID_ARG;
    const int esz = dtype == MOEGG_BF16 ? 2 : 1;
    const bool w4 = dtype == MOEGG_FP8_E4M3_FP4_E2M1;
    if (dtype != MOEGG_BF16) {
        if (!A_scale || !B_scale) return MOEGG_ERR_INVALID_ARG;
        if (!aligned(A_scale, 4) || !aligned(B_scale, 4)) return MOEGG_ERR_INVALID_ARG;
    }
    // packed E2M1 is [G, N, K/2] or its panels [G, N/P, K/128, P, 64]
    if (w4 && b_layout != MOEGG_B_NK && b_layout != MOEGG_B_NK_PANEL) return MOEGG_ERR_UNSUPPORTED;
    // E8M0 scale rows are read four bytes at a time: N / 128 bytes per weight-scale row
    if (e8m0_scales(dtype) && (N % 512 != 0 || N / 128 > 256)) return MOEGG_ERR_UNSUPPORTED;
    if (K % (128 / esz) != 0 || N % col_tile != 0) return MOEGG_ERR_UNSUPPORTED;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16)) return MOEGG_ERR_INVALID_ARG;
    if ((w4 ? (int64_t)K * N / 2 : (int64_t)K * N * esz) > kMaxBufferBytes) return MOEGG_ERR_UNSUPPORTED;
    return MOEGG_OK;
}

}  // namespace

extern "C" {

int moegg_version(void) { return (0 << 16) | 1; }

const char* moegg_status_string(moegg_status_t s) {
    switch (s) {
        case MOEGG_OK: return "ok";
        case MOEGG_ERR_INVALID_ARG: return "invalid argument";
        case MOEGG_ERR_UNSUPPORTED: return "unsupported shape or option";
        case MOEGG_ERR_WORKSPACE: return "workspace missing or too small";
        case MOEGG_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t moegg_workspace_bytes(int G, int64_t max_rows) {
    if (G < 1 || G > kMaxExperts || max_rows < 0) return 0;
    return ws_layout(G, max_rows).total;
}

static bool valid_block_m(int b) {
    return b == 0 || b == 64 || b == 128 || b == 256 || b == MOEGG_BLOCK_M_PER_EXPERT;
}

moegg_status_t moegg_schedule(const int32_t* m_sizes, int G, int64_t rows_total, int seg_align, int block_m,
                              int N, void* ws, size_t ws_bytes, void* stream) {
    if (!m_sizes || G < 1 || G > kMaxExperts || rows_total < 0 || rows_total > INT32_MAX || seg_align < 1)
        return MOEGG_ERR_INVALID_ARG;
    if (!valid_block_m(block_m)) return MOEGG_ERR_UNSUPPORTED;
    if (!ws || !aligned(ws, 256)) return MOEGG_ERR_WORKSPACE;
    const WsLayout L = ws_layout(G, rows_total);
    if (ws_bytes < L.total) return MOEGG_ERR_WORKSPACE;
    if (N < 1) return MOEGG_ERR_INVALID_ARG;
    const int n_col_tiles = N / 256 > 0 ? N / 256 : 1;
    return hip_status(launch_sched(m_sizes, G, rows_total, seg_align, 0, 0, block_m, n_col_tiles, 0, ws,
                                   L.max_tiles, (hipStream_t)stream),
                      "schedule");
}

moegg_status_t moegg_schedule_exemplar(const int32_t* m_sizes, int G, int64_t rows_total, int seg_align, int N,
                                       const moegg_exemplar_t* exemplars, int n_exemplars, int hysteresis,
                                       void* ws, size_t ws_bytes, void* stream) {
    if (!m_sizes || !aligned(m_sizes, 4) || G < 1 || G > kMaxExperts || rows_total < 0 || rows_total > INT32_MAX ||
        seg_align < 1 || N < 1)
        return MOEGG_ERR_INVALID_ARG;
    if (!exemplars || !aligned(exemplars, 4) || n_exemplars < 1 || hysteresis < 0) return MOEGG_ERR_INVALID_ARG;
    if (n_exemplars > MOEGG_MAX_EXEMPLARS) return MOEGG_ERR_UNSUPPORTED;
    if (!ws || !aligned(ws, 256)) return MOEGG_ERR_WORKSPACE;
    const WsLayout L = ws_layout(G, rows_total);
    if (ws_bytes < L.total) return MOEGG_ERR_WORKSPACE;
    // the cost rule (used if an exemplar names no valid height) counts 256-wide column tiles
    const int n_col_tiles = N / 256 > 0 ? N / 256 : 1;
    return hip_status(launch_sched_exemplar(m_sizes, G, rows_total, seg_align, n_col_tiles, exemplars, n_exemplars,
                                            hysteresis, ws, L.max_tiles, (hipStream_t)stream),
                      "exemplar schedule");
}

moegg_status_t moegg_selection_read(const void* ws, moegg_selection_t* h_out, void* stream) {
    if (!ws || !h_out) return MOEGG_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    Control ctl;
    hipError_t e = hipMemcpyAsync(&ctl, (const char*)ws + 128, sizeof(ctl), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "selection read");
    if (ctl.sel_tag != kSelectorTag) return MOEGG_ERR_INVALID_ARG;
    h_out->exemplar = ctl.sel_prev;
    h_out->size_class = ctl.sel_size_class;
    for (int q = 0; q < 8; ++q) h_out->lorenz[q] = ctl.sel_lorenz[q];
    h_out->distance = ctl.sel_distance;
    return MOEGG_OK;
}

}  // extern "C"

namespace {

// Argument checks of the contiguous call, everything but the workspace.
moegg_status_t check_contiguous(const void* A, const void* A_scale, const void* B, const void* B_scale,
                                const void* C, const int32_t* m_sizes, int G, int64_t rows_total, int K, int N,
                                int seg_align, moegg_dtype_t dtype, moegg_b_layout_t b_layout, int block_m) {
    if (!m_sizes || !aligned(m_sizes, 4)) return MOEGG_ERR_INVALID_ARG;
    moegg_status_t st = check_common(A, A_scale, B, B_scale, C, G, K, N, dtype, b_layout, 256);
    if (st != MOEGG_OK) return st;
    if (rows_total < 0 || rows_total > INT32_MAX || seg_align < 1) return MOEGG_ERR_INVALID_ARG;
    if (e8m0_scales(dtype) && rows_total % 4 != 0) return MOEGG_ERR_UNSUPPORTED;
    if (!transposed_scales_fit(dtype, K / 128, rows_total)) return MOEGG_ERR_UNSUPPORTED;
    if (!valid_block_m(block_m)) return MOEGG_ERR_UNSUPPORTED;
    const int esz = dtype == MOEGG_BF16 ? 2 : 1;
    if (256ll * K * esz > kMaxBufferBytes || 256ll * N * 2 > kMaxBufferBytes) return MOEGG_ERR_UNSUPPORTED;
    return MOEGG_OK;
}

// Scheduler + contiguous GEMM on a checked problem, with the workspace at ws.
moegg_status_t launch_contiguous_call(const void* A, const void* A_scale, const void* B, const void* B_scale,
                                      void* C, const int32_t* m_sizes, int G, int64_t rows_total, int K, int N,
                                      int seg_align, moegg_dtype_t dtype, moegg_b_layout_t b_layout, int block_m,
                                      void* ws, hipStream_t s) {
    const WsLayout L = ws_layout(G, rows_total);
    hipError_t e = launch_sched(m_sizes, G, rows_total, seg_align, 0, 0, block_m, N / 256, 0, ws, L.max_tiles, s);
    if (e != hipSuccess) return hip_status(e, "scheduler launch");
    ContigArgs a{A, A_scale, B, B_scale, C, m_sizes, (const unsigned char*)ws, G, K, N, 0, (int)rows_total};
    a.a_scale_km = dtype == MOEGG_FP8_E4M3_SCALE_KM;
    a.b_panel = layout_panel(b_layout);
    e = launch_contiguous(a, dtype != MOEGG_BF16, e8m0_scales(dtype), dtype == MOEGG_FP8_E4M3_FP4_E2M1,
                          layout_kn(b_layout), rows_total, block_m, s);
    if (debug_on())
        fprintf(stderr, "moegg: contiguous G=%d rows=%lld K=%d N=%d align=%d dtype=%d b_layout=%d block_m=%d\n", G,
                (long long)rows_total, K, N, seg_align, (int)dtype, (int)b_layout, block_m);
    return hip_status(e, "contiguous GEMM launch");
}

}  // namespace

// ------------------------------------------------------------ allocation-free variant
//
// The workspace of moegg_grouped_gemm_contiguous_noalloc: a fixed array in
// each GPU's memory, for callers that cannot allocate.  In host code the
// name `scratch` is only a stand-in for the symbol; its device address on a
// GPU comes from hipGetSymbolAddress with that GPU current, looked up once per
// GPU and kept in scratch_ptr, and only that address is ever handed to a
// kernel.  Calls on one GPU share the array: the scheduler writes every field
// the GEMM reads (stats, control block, offsets, tile list) before the GEMM
// runs, so nothing needs clearing, but calls that overlap on one GPU race.
namespace {
constexpr size_t kNoAllocScratchBytes = MOEGG_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// Device address of `scratch` on the calling thread's current GPU.
hipError_t scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

extern "C" {

moegg_status_t moegg_grouped_gemm_contiguous(const void* A, const void* A_scale, const void* B,
                                             const void* B_scale, void* C, const int32_t* m_sizes, int G,
                                             int64_t rows_total, int K, int N, int seg_align,
                                             moegg_dtype_t dtype, moegg_b_layout_t b_layout, int block_m,
                                             void* ws, size_t ws_bytes, void* stream) {
    moegg_status_t st = check_contiguous(A, A_scale, B, B_scale, C, m_sizes, G, rows_total, K, N, seg_align, dtype,
                                         b_layout, block_m);
    if (st != MOEGG_OK) return st;
    if (!ws || !aligned(ws, 256)) return MOEGG_ERR_WORKSPACE;
    if (ws_bytes < ws_layout(G, rows_total).total) return MOEGG_ERR_WORKSPACE;
    return launch_contiguous_call(A, A_scale, B, B_scale, C, m_sizes, G, rows_total, K, N, seg_align, dtype,
                                  b_layout, block_m, ws, (hipStream_t)stream);
}

moegg_status_t moegg_grouped_gemm_contiguous_noalloc(const void* A, const void* A_scale, const void* B,
                                                     const void* B_scale, void* C, const int32_t* m_sizes, int G,
                                                     int64_t rows_total, int K, int N, int seg_align,
                                                     moegg_dtype_t dtype, moegg_b_layout_t b_layout, int block_m,
                                                     void* stream) {
    moegg_status_t st = check_contiguous(A, A_scale, B, B_scale, C, m_sizes, G, rows_total, K, N, seg_align, dtype,
                                         b_layout, block_m);
    if (st != MOEGG_OK) return st;
    if (ws_layout(G, rows_total).total > kNoAllocScratchBytes) return MOEGG_ERR_WORKSPACE;
    void* ws = nullptr;
    hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) return hip_status(e, "scratch lookup");
    return launch_contiguous_call(A, A_scale, B, B_scale, C, m_sizes, G, rows_total, K, N, seg_align, dtype,
                                  b_layout, block_m, ws, (hipStream_t)stream);
}

moegg_status_t moegg_grouped_gemm_contiguous_scheduled(const void* A, const void* A_scale, const void* B,
                                                       const void* B_scale, void* C, int G, int64_t rows_total,
                                                       int K, int N, moegg_dtype_t dtype,
                                                       moegg_b_layout_t b_layout, int block_m, const void* ws,
                                                       size_t ws_bytes, void* stream) {
    moegg_status_t st = check_common(A, A_scale, B, B_scale, C, G, K, N, dtype, b_layout, 256);
    if (st != MOEGG_OK) return st;
    if (rows_total < 0 || rows_total > INT32_MAX) return MOEGG_ERR_INVALID_ARG;
    if (e8m0_scales(dtype) && rows_total % 4 != 0) return MOEGG_ERR_UNSUPPORTED;
    if (!transposed_scales_fit(dtype, K / 128, rows_total)) return MOEGG_ERR_UNSUPPORTED;
    if (!valid_block_m(block_m)) return MOEGG_ERR_UNSUPPORTED;
    const int esz = dtype == MOEGG_BF16 ? 2 : 1;
    if (256ll * K * esz > kMaxBufferBytes || 256ll * N * 2 > kMaxBufferBytes) return MOEGG_ERR_UNSUPPORTED;
    if (!ws || !aligned(ws, 256)) return MOEGG_ERR_WORKSPACE;
    if (ws_bytes < ws_layout(G, rows_total).total) return MOEGG_ERR_WORKSPACE;
    ContigArgs a{A, A_scale, B, B_scale, C, nullptr, (const unsigned char*)ws, G, K, N, 0, (int)rows_total};
    a.a_scale_km = dtype == MOEGG_FP8_E4M3_SCALE_KM;
    a.b_panel = layout_panel(b_layout);
    return hip_status(launch_contiguous(a, dtype != MOEGG_BF16, e8m0_scales(dtype), dtype == MOEGG_FP8_E4M3_FP4_E2M1,
                                        layout_kn(b_layout), rows_total, block_m, (hipStream_t)stream),
                      "scheduled contiguous GEMM launch");
}

moegg_status_t moegg_grouped_gemm_swiglu_scheduled(const void* A, const void* A_scale, const void* W1,
                                                   const void* W1_scale, void* H, void* H_scale, int G,
                                                   int64_t rows_total, int K, int I, moegg_dtype_t dtype,
                                                   moegg_b_layout_t b_layout, int block_m, const void* ws,
                                                   size_t ws_bytes, void* stream) {
    if (I < 1 || (int64_t)I * 2 > INT32_MAX) return MOEGG_ERR_INVALID_ARG;
    if (H_scale && !aligned(H_scale, 4)) return MOEGG_ERR_INVALID_ARG;
    const int N = 2 * I;
    moegg_status_t st = check_common(A, A_scale, W1, W1_scale, H, G, K, N, dtype, b_layout, 256);
    if (st != MOEGG_OK) return st;
    if (dtype == MOEGG_FP8_E4M3_E8M0) return MOEGG_ERR_UNSUPPORTED;
    if (dtype == MOEGG_FP8_E4M3_FP4_E2M1 && rows_total % 4 != 0) return MOEGG_ERR_UNSUPPORTED;
    // A_scale [K/128, rows_total] in; with MOEGG_FP8_E4M3_SCALE_KM also H_scale [I/128, rows_total] out
    if (!transposed_scales_fit(dtype, std::max(K, I) / 128, rows_total)) return MOEGG_ERR_UNSUPPORTED;
    if (b_layout != MOEGG_B_NK && b_layout != MOEGG_B_NK_PANEL) return MOEGG_ERR_UNSUPPORTED;
    if (rows_total < 0 || rows_total > INT32_MAX) return MOEGG_ERR_INVALID_ARG;
    if (!valid_block_m(block_m)) return MOEGG_ERR_UNSUPPORTED;
    const int esz = dtype == MOEGG_BF16 ? 2 : 1;
    if (256ll * K * esz > kMaxBufferBytes || 256ll * N > kMaxBufferBytes) return MOEGG_ERR_UNSUPPORTED;
    if (!ws || !aligned(ws, 256)) return MOEGG_ERR_WORKSPACE;
    if (ws_bytes < ws_layout(G, rows_total).total) return MOEGG_ERR_WORKSPACE;
    ContigArgs a{A, A_scale, W1, W1_scale, H, nullptr, (const unsigned char*)ws, G, K, N, 0, (int)rows_total,
                 H_scale};
    a.a_scale_km = dtype == MOEGG_FP8_E4M3_SCALE_KM;
    a.b_panel = layout_panel(b_layout);
    return hip_status(launch_contiguous_swiglu(a, dtype != MOEGG_BF16, dtype == MOEGG_FP8_E4M3_FP4_E2M1, rows_total,
                                               block_m, (hipStream_t)stream),
                      "SwiGLU GEMM launch");
}

moegg_status_t moegg_expert_mlp_fused(const void* A, const float* A_scale, const void* W1, const float* W1_scale,
                                     const void* W2, const float* W2_scale, void* H, float* H_scale, void* Y,
                                     const int32_t* m_sizes, int G, int64_t rows_total, int K, int I, int N2,
                                     int seg_align, moegg_dtype_t dtype, moegg_b_layout_t b_layout, void* ws,
                                     size_t ws_bytes, void* stream) {
    if (!m_sizes || !aligned(m_sizes, 4) || seg_align < 1) return MOEGG_ERR_INVALID_ARG;
    if (I < 1 || (int64_t)I * 2 > INT32_MAX || N2 < 1) return MOEGG_ERR_INVALID_ARG;
    if (dtype != MOEGG_FP8_E4M3 && dtype != MOEGG_FP8_E4M3_SCALE_KM) return MOEGG_ERR_UNSUPPORTED;
    if (b_layout != MOEGG_B_NK && b_layout != MOEGG_B_NK_PANEL) return MOEGG_ERR_UNSUPPORTED;
    if (!H_scale || !aligned(H_scale, 4)) return MOEGG_ERR_INVALID_ARG;
    if (rows_total < 0 || rows_total > INT32_MAX) return MOEGG_ERR_INVALID_ARG;
    // L1: A [rows, K] x W1 [G, 2I, K] -> H; L2: H [rows, I] x W2 [G, N2, I] -> Y
    moegg_status_t st = check_common(A, A_scale, W1, W1_scale, H, G, K, 2 * I, dtype, b_layout, 256);
    if (st != MOEGG_OK) return st;
    st = check_common(H, H_scale, W2, W2_scale, Y, G, I, N2, dtype, b_layout, 256);
    if (st != MOEGG_OK) return st;
    if (!transposed_scales_fit(dtype, std::max(K, I) / 128, rows_total)) return MOEGG_ERR_UNSUPPORTED;
    if (256ll * std::max(K, I) > kMaxBufferBytes || 256ll * std::max(2 * I, 2 * N2) > kMaxBufferBytes)
        return MOEGG_ERR_UNSUPPORTED;
    if (!ws || !aligned(ws, 256)) return MOEGG_ERR_WORKSPACE;
    const WsLayout L = ws_layout(G, rows_total);
    if (ws_bytes < L.total) return MOEGG_ERR_WORKSPACE;
    // at most ceil(rows_total / 256) + G row tiles at the 256-row height
    const int64_t max_rt = (rows_total + 255) / 256 + G;
    const int64_t blocks = mlp_blocks(max_rt, 2 * I / 256, N2 / 256);
    if (blocks > INT32_MAX) return MOEGG_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    // the scheduler also clears the completion counters (no memset node under graph capture)
    uint32_t* sync = (uint32_t*)((unsigned char*)ws + L.sync);
    hipError_t e = launch_sched(m_sizes, G, rows_total, seg_align, 0, 0, 256, 2 * I / 256, 0, ws, L.max_tiles, s,
                                sync, L.max_tiles);
    if (e != hipSuccess) return hip_status(e, "scheduler launch");
    MlpArgs a{};
    a.l1 = ContigArgs{A, A_scale, W1, W1_scale, H, nullptr, (const unsigned char*)ws, G, K, 2 * I, 0,
                      (int)rows_total, H_scale};
    a.l2 = ContigArgs{H, H_scale, W2, W2_scale, Y, nullptr, (const unsigned char*)ws, G, I, N2, 0, (int)rows_total};
    a.l1.a_scale_km = a.l2.a_scale_km = dtype == MOEGG_FP8_E4M3_SCALE_KM;
    a.l1.b_panel = a.l2.b_panel = layout_panel(b_layout);
    a.sync = sync;
    a.l1_blocks = (int)mlp_l1_blocks(max_rt, 2 * I / 256);
    e = launch_mlp_fused(a, (int)blocks, s);
    if (debug_on())
        fprintf(stderr, "moegg: expert MLP fused G=%d rows=%lld K=%d I=%d N2=%d dtype=%d b_layout=%d blocks=%lld\n", G,
                (long long)rows_total, K, I, N2, (int)dtype, (int)b_layout, (long long)blocks);
    return hip_status(e, "fused expert MLP launch");
}

moegg_status_t moegg_grouped_gemm_masked(const void* A, const void* A_scale, const void* B, const void* B_scale,
                                         void* C, const int32_t* masked_m, int G, int cap, int K, int N,
                                         moegg_dtype_t dtype, moegg_b_layout_t b_layout, void* ws,
                                         size_t ws_bytes, void* stream) {
    if (!masked_m || !aligned(masked_m, 4)) return MOEGG_ERR_INVALID_ARG;
    moegg_status_t st = check_common(A, A_scale, B, B_scale, C, G, K, N, dtype, b_layout, masked_block_n());
    if (st != MOEGG_OK) return st;
    if (cap < 1 || (int64_t)G * cap > INT32_MAX) return MOEGG_ERR_INVALID_ARG;
    // E8M0 activation scales [K/128, G * cap] are read four bytes at a time
    if (e8m0_scales(dtype) && ((int64_t)G * cap) % 4 != 0) return MOEGG_ERR_UNSUPPORTED;
    if (!transposed_scales_fit(dtype, K / 128, (int64_t)G * cap)) return MOEGG_ERR_UNSUPPORTED;
    const int esz = dtype == MOEGG_BF16 ? 2 : 1;
    if ((int64_t)masked_block_m() * K * esz > kMaxBufferBytes) return MOEGG_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (ws) {
        if (!aligned(ws, 256)) return MOEGG_ERR_WORKSPACE;
        const WsLayout L = ws_layout(G, (int64_t)G * cap);
        if (ws_bytes < L.total) return MOEGG_ERR_WORKSPACE;
        e = launch_sched(masked_m, G, (int64_t)G * cap, 1, cap, 1, 0, N / masked_block_n(), masked_block_m(), ws,
                         L.max_tiles, s);
        if (e != hipSuccess) return hip_status(e, "masked stats launch");
    }
    ContigArgs a{A, A_scale, B, B_scale, C, masked_m, (const unsigned char*)ws, G, K, N, cap, G * cap};
    a.a_scale_km = dtype == MOEGG_FP8_E4M3_SCALE_KM;
    a.b_panel = layout_panel(b_layout);
    e = launch_masked(a, dtype != MOEGG_BF16, e8m0_scales(dtype), dtype == MOEGG_FP8_E4M3_FP4_E2M1,
                      layout_kn(b_layout), s);
    return hip_status(e, "masked GEMM launch");
}

// Shared by the bf16 and fp8 K-grouped calls.  fp8: e4m3 operands with scales, fp32 or (e8m0) exponent bytes.
static moegg_status_t k_grouped_call(const void* X, const void* X_scale, const void* dY, const void* dY_scale,
                                     float* dW, const int32_t* t_sizes, int G, int64_t T, int Mw, int Nw,
                                     int64_t scale_groups, bool fp8, bool e8m0, void* ws, size_t ws_bytes,
                                     void* stream) {
    // with T = 0 no row is read, so X and dY may be NULL (an empty tensor's pointer)
    if ((T > 0 && (!X || !dY)) || !dW || !t_sizes) return MOEGG_ERR_INVALID_ARG;
    if (G < 1 || G > kMaxExperts || T < 0 || Mw < 1 || Nw < 1) return MOEGG_ERR_INVALID_ARG;
    if (Mw % 256 != 0 || Nw % 256 != 0) return MOEGG_ERR_UNSUPPORTED;
    if (!aligned(X, 16) || !aligned(dY, 16) || !aligned(dW, 16) || !aligned(t_sizes, 4))
        return MOEGG_ERR_INVALID_ARG;
    const int64_t esz = fp8 ? 1 : 2;
    if (T * Mw * esz > kMaxBufferBytes || T * Nw * esz > kMaxBufferBytes) return MOEGG_ERR_UNSUPPORTED;
    if (fp8) {
        if (scale_groups < 0 || (T > 0 && (scale_groups < 1 || !X_scale || !dY_scale))) return MOEGG_ERR_INVALID_ARG;
        if (!aligned(X_scale, 4) || !aligned(dY_scale, 4)) return MOEGG_ERR_INVALID_ARG;
        // scale offsets are 32-bit; the parked offset 2^31 must lie past both arrays
        if (scale_groups * (int64_t)std::max(Mw, Nw) * (e8m0 ? 1 : 4) >= 0x80000000ll) return MOEGG_ERR_UNSUPPORTED;
    }
    if (!ws || !aligned(ws, 256)) return MOEGG_ERR_WORKSPACE;
    const WsLayout L = ws_layout(G, 0);
    if (ws_bytes < L.total) return MOEGG_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_sched_k_grouped(t_sizes, G, T, fp8 ? scale_groups : 0, ws, s);
    if (e != hipSuccess) return hip_status(e, "K-grouped scheduler launch");
    KGroupedArgs a{X, dY, dW, (const unsigned char*)ws, G, Mw, Nw, X_scale, dY_scale, scale_groups};
    return hip_status(launch_k_grouped(a, fp8, e8m0, s), "K-grouped GEMM launch");
}

moegg_status_t moegg_grouped_gemm_k_grouped(const void* X, const void* dY, float* dW, const int32_t* t_sizes, int G,
                                            int64_t T, int Mw, int Nw, void* ws, size_t ws_bytes, void* stream) {
    return k_grouped_call(X, nullptr, dY, nullptr, dW, t_sizes, G, T, Mw, Nw, 0, false, false, ws, ws_bytes,
                          stream);
}

moegg_status_t moegg_grouped_gemm_k_grouped_fp8(const void* X, const float* X_scale, const void* dY,
                                                const float* dY_scale, float* dW, const int32_t* t_sizes, int G,
                                                int64_t T, int Mw, int Nw, int64_t scale_groups, void* ws,
                                                size_t ws_bytes, void* stream) {
    return k_grouped_call(X, X_scale, dY, dY_scale, dW, t_sizes, G, T, Mw, Nw, scale_groups, true, false, ws,
                          ws_bytes, stream);
}

moegg_status_t moegg_grouped_gemm_k_grouped_e8m0(const void* X, const uint8_t* X_scale, const void* dY,
                                                 const uint8_t* dY_scale, float* dW, const int32_t* t_sizes, int G,
                                                 int64_t T, int Mw, int Nw, int64_t scale_groups, void* ws,
                                                 size_t ws_bytes, void* stream) {
    return k_grouped_call(X, X_scale, dY, dY_scale, dW, t_sizes, G, T, Mw, Nw, scale_groups, true, true, ws,
                          ws_bytes, stream);
}

moegg_status_t moegg_stats_report(const moegg_stats_t* h_stats, moegg_report_t* h_out) {
    if (!h_stats || !h_out) return MOEGG_ERR_INVALID_ARG;
    const moegg_stats_t& st = *h_stats;
    if (st.U < 0 || st.sum_sq < 0 || st.P_exec < 0) return MOEGG_ERR_INVALID_ARG;
    for (int i = 0; i < MOEGG_NUM_Q; ++i)
        if (st.P_at[i] < 0) return MOEGG_ERR_INVALID_ARG;
    // U <= 2^31, so U^2 and every difference below are exact in a 64-bit mantissa
    auto ratio = [](long double num, long double den) -> double {
        return den == 0 ? 0.0 : (double)(num / den);
    };
    const long double U = (long double)st.U;
    h_out->effective_experts = ratio(U * U, (long double)st.sum_sq);
    for (int i = 0; i < MOEGG_NUM_Q; ++i) {
        const long double P = (long double)st.P_at[i];
        h_out->padding_fraction[i] = ratio(P - U, P);
        h_out->useful_share[i] = ratio(U, P);
    }
    h_out->exec_padding_fraction = ratio((long double)st.P_exec - U, (long double)st.P_exec);
    h_out->physical_over_effective = ratio((long double)st.P_exec, U);
    return MOEGG_OK;
}

moegg_status_t moegg_stats_read(const void* ws, moegg_stats_t* h_out, void* stream) {
    if (!ws || !h_out) return MOEGG_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(h_out, ws, sizeof(moegg_stats_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return hip_status(e, "stats read");
}

moegg_status_t moegg_tile_list_read(const void* ws, moegg_tile_t* h_tiles, int64_t cap_tiles, int64_t* h_n,
                                    void* stream) {
    if (!ws || !h_n || cap_tiles < 0 || (cap_tiles > 0 && !h_tiles)) return MOEGG_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    Control ctl;
    hipError_t e = hipMemcpyAsync(&ctl, (const char*)ws + 128, sizeof(ctl), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "tile count read");
    *h_n = ctl.n_tiles;
    int64_t n = ctl.n_tiles < cap_tiles ? ctl.n_tiles : cap_tiles;
    if (n > 0) {
        const WsLayout L = ws_layout(ctl.G, 0);
        e = hipMemcpyAsync(h_tiles, (const char*)ws + L.tiles, sizeof(moegg_tile_t) * (size_t)n,
                           hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_status(e, "tile list read");
    }
    return MOEGG_OK;
}

}  // extern "C"
