// gemm.hip -- MoE grouped GEMM kernels for gfx950 (CDNA4).
//
// Layouts, from the DeepGEMM grouped/masked MoE GEMM record ("Workarounds"):
//   - M-grouped contiguous: each expert's rows back to back in A; the work
//     list comes from the device scheduler.
//   - masked: a capacity buffer [G, cap, K] plus per-expert valid counts,
//     read at run time, with a fixed grid for graph replay.
//   - K-grouped weight gradient: the reduction axis is split by expert.
// Grouping alters only how the work is tiled, not what each output is (same
// record, "Arithmetic intensity"): every valid output is a plain dot product
// over K, accumulated in fp32.
//
// Kernel structure (one 512-thread workgroup per output tile):
//   - Stage loads go straight from HBM to LDS (buffer_load_dwordx4 ... lds).
//     Each buffer resource covers only the tile's valid rows, so padding rows
//     read as zeros and cost no HBM traffic.
//   - Every LDS row holds 128 bytes of K: 128 e4m3 values or 64 bf16.  One
//     such stage feeds one 16x16x128 fp8 MFMA, or two 16x16x32 bf16 MFMAs.
//   - An operand stored K-contiguous is read with ds_read_b128.  An operand
//     stored N/M-contiguous ([K, N] weights, K-grouped X and dY) is staged
//     as-is and transposed on the way out of LDS with ds_read_b64_tr_b8/_b16.
//   - XOR swizzles on 16-byte chunks keep the DMA writes and the fragment
//     reads free of bank conflicts.
//   - The weight tile is the MFMA A operand and the activation tile the B
//     operand.  So each lane ends with 4 consecutive output columns of one
//     row: one per-row fp8 scale per lane, and 8-byte (bf16) or 16-byte
//     (fp32) stores.
//   - Tail padding: a tile skips every 16-row MFMA block that lies wholly
//     past its valid rows ("Grouped execution does not require padded
//     experts" on the MoE GroupGEMM padding page keeps tail padding inside
//     an MMA tile; here it shrinks to the 16-row MFMA block).
//   - fp8: each 128-wide K group's fp32 MFMA partial is promoted into the
//     fp32 accumulator with acc += partial * a_scale[row] * b_scale[block].
//   - Tile order is XCD-aware.  Block b runs on XCD b % 8, and each XCD
//     takes runs of 32 consecutive work items: 4 row tiles x 8 column tiles
//     of one expert, which share A tiles and weight panels in that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"
#include "workspace.hpp"
#include "tile_order.hpp"

namespace moegg {

template <int X> struct dependent_false { static constexpr bool value = false; };

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Swizzle of 16-byte chunks in a K-contiguous tile (128-byte rows), by element
// size.  A fragment read has lane (r = l % 16, g = l / 16) fetch chunk 2g + h
// (e4m3) or 4kk + g (bf16) of row r.  Measured on gfx950 with 8 waves per CU
// (SQ_LDS_BANK_CONFLICT against SQ_LDS_IDX_ACTIVE): these two swizzles make
// their reads take 4 LDS cycles per 1 KB (no bank conflicts); exchanging
// them, or XOR-ing row & 7, costs 8.
template <int ESZ>
__device__ __forceinline__ int swz_k(int row) {
    if constexpr (ESZ == 1) return ((row & 3) << 1) | ((row >> 2) & 1);
    else return (row >> 1) & 7;
}

// Swizzle of 16-byte chunks in an MN-contiguous tile, by element size and
// row bytes, chosen so the 16 lanes of one transpose read hit distinct banks.
template <int ESZ, int RB>
__device__ __forceinline__ int swz_mn(int k) {
    if constexpr (ESZ == 1 && RB == 256) return (k & 7) | (((k >> 5) & 1) << 3);
    else if constexpr (ESZ == 1 && RB == 128) return ((k >> 1) & 3) | (((k >> 5) & 1) << 2);
    else if constexpr (ESZ == 2 && (RB == 512 || RB == 256)) return ((k & 3) << 1) | (((k >> 3) & 1) << 3);
    else if constexpr (ESZ == 2 && RB == 128) return (((k >> 1) & 1) << 1) | (((k >> 3) & 1) << 2);
    else static_assert(dependent_false<RB>::value, "unsupported MN tile row size");
    return 0;
}

// Tile configuration of the K-grouped weight gradient (both operands
// M/N-contiguous): 512 threads as WAVES_M x WAVES_N waves over a BM x BN tile
// of dW; a stage holds KSTEP rows of the reduction axis of both operands (128
// bytes of each column: 64 bf16 rows, or 128 e4m3 rows = one scale group), and
// with fp8 the group's scales of the tile's columns, [X scales | dY scales]:
// fp32, or (E8M0) exponent bytes that the MFMA applies itself.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, bool FP8_ = false, bool E8M0_ = false>
struct KCfg {
    static constexpr bool FP8 = FP8_;
    static constexpr bool E8M0 = E8M0_;
    static constexpr int ESZ = FP8 ? 1 : 2;
    static constexpr int KSTEP = 128 / ESZ;            // reduction rows per stage
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int STAGES = STAGES_;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;   // wave tile
    static constexpr int MB = WTM / 16, NB = WTN / 16;             // 16x16 blocks per wave
    static constexpr int A_BYTES = BM * KSTEP * ESZ;
    static constexpr int B_BYTES = BN * KSTEP * ESZ;
    static constexpr int S_BYTES = FP8 ? (BM + BN) * (E8M0 ? 1 : 4) : 0;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_LOADS = A_BYTES / 16 / THREADS;         // 16-byte DMAs per thread per stage
    static constexpr int B_LOADS = B_BYTES / 16 / THREADS;
    static constexpr int OPS = A_LOADS + B_LOADS + (FP8 ? 1 : 0);  // fp8: one 4-byte scale DMA
    static_assert(A_BYTES % (16 * THREADS) == 0 && B_BYTES % (16 * THREADS) == 0, "stage split");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    static_assert(!FP8 || E8M0 || BM + BN == THREADS, "one scale per thread per stage");
    static_assert(!E8M0 || (FP8 && BM == 256 && BN == 256 && WAVES % 2 == 0), "E8M0: 256 scale bytes per wave");
    static_assert(STAGES >= 2 && LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(OPS * (STAGES - 2) < 64, "vmcnt range");
};

// ---------------------------------------------------------------- stage loads

// One DMA of an MN-contiguous tile: KSTEP rows (one per K index) of RB bytes,
// from a buffer whose K row k starts at k * row_bytes, column byte cbyte.
template <class C, int RB>
__device__ __forceinline__ void load_mn_one(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, uint32_t k0,
                                            uint32_t cbyte, char* lds_tile, int j) {
    const int tid = threadIdx.x, wave = tid >> 6;
    constexpr int CPR = RB / 16;                       // chunks per row
    const int f = j * C::THREADS + tid;
    const int r = f / CPR, p = f % CPR;
    const int c = p ^ swz_mn<C::ESZ, RB>(r);
    load16_to_lds(rs, (k0 + r) * row_bytes + cbyte + c * 16, lds_tile + (j * C::THREADS + wave * 64) * 16);
}

template <class C, int RB>
__device__ __forceinline__ void load_tile_mn(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, uint32_t k0,
                                             uint32_t cbyte, char* lds_tile, int loads) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j >= loads) break;
        load_mn_one<C, RB>(rs, row_bytes, k0, cbyte, lds_tile, j);
    }
}

// ---------------------------------------------------------------- fragments

// K-contiguous tile, fp8: lane (row r16, group g) gets bytes [32g, 32g+32).
__device__ __forceinline__ v8i frag_k_fp8(const char* tile, int row) {
    const int g = (threadIdx.x & 63) >> 4;
    const int s = swz_k<1>(row);
    v4i lo = lds_read_b128(tile + row * 128 + (((2 * g) ^ s) << 4));
    v4i hi = lds_read_b128(tile + row * 128 + (((2 * g + 1) ^ s) << 4));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// K-contiguous tile, fp8, in the MFMA's own K order: lane (row r16, group g)
// gets bytes [16g, 16g+16) and [64+16g, 64+16g+16).  Measured on gfx950 with
// one-hot operands: the 16x16x128 MFMA takes an e4m3 operand's 32 bytes per
// lane as k = 16g + (0..15), then 64 + 16g + (0..15), but an E2M1 operand's
// 16 bytes as k = 32g + (0..31).  Two e4m3 operands read alike (frag_k_fp8)
// pair up whatever the order; against fp4 weights the activations are read
// this way.
__device__ __forceinline__ v8i frag_k_fp8_mfma_order(const char* tile, int row) {
    const int g = (threadIdx.x & 63) >> 4;
    const int s = swz_k<1>(row);
    v4i lo = lds_read_b128(tile + row * 128 + ((g ^ s) << 4));
    v4i hi = lds_read_b128(tile + row * 128 + (((g + 4) ^ s) << 4));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// K-contiguous tile, bf16, half-step kk: lane gets k = 32kk + 8g + (0..7).
__device__ __forceinline__ v4i frag_k_bf16(const char* tile, int row, int kk) {
    const int g = (threadIdx.x & 63) >> 4;
    return lds_read_b128(tile + row * 128 + (((4 * kk + g) ^ swz_k<2>(row)) << 4));
}

// Swizzle of 16-byte chunks in a K-contiguous fp4 weight tile (64-byte rows:
// 128 E2M1 values, two per byte).  A fragment read has lane (r = l % 16,
// g = l / 16) fetch chunk g of row r; XOR-ing it with bits 1..2 of the row,
// flipped by bit 3, puts the 16 rows a chunk index is read from on 16
// distinct 16-byte slots of 256 bytes, and any 8 consecutive rows on 8
// distinct slots of 128 bytes.
__device__ __forceinline__ int swz_w4(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// K-contiguous fp4 tile: lane (row r16, group g) gets the 16 bytes holding
// k = 32g + (0..31), element 2i in the low nibble of byte i -- the E2M1
// operand layout of the 16x16x128 MFMA (8 values per register, lowest
// nibble first).  The upper half of the operand is unused for fp4.
__device__ __forceinline__ v8i frag_k_fp4(const char* tile, int row) {
    const int g = (threadIdx.x & 63) >> 4;
    v4i v = lds_read_b128(tile + row * 64 + ((g ^ swz_w4(row)) << 4));
    return v8i{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
}

// MN-contiguous tile, fp8: lane (col n0 + l%16, group g) gets the 32 bytes
// k = 32g + (0..31) of column n, via four tr8 reads of 8 K rows each.
template <int RB>
__device__ __forceinline__ v8i frag_mn_fp8(const char* tile, int n0) {
    const int lane = threadIdx.x & 63, g = lane >> 4, s = lane & 15;
    const int c = n0 >> 4;               // 16-byte chunk of columns n0..n0+15
    v2i part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int k = 32 * g + 8 * j + (s >> 1);
        part[j] = lds_read_tr8(tile + k * RB + ((c ^ swz_mn<1, RB>(k)) << 4) + 8 * (s & 1));
    }
    return v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
}

// MN-contiguous tile, bf16, half-step kk: lane gets k = 32kk + 8g + (0..7)
// of column n0 + l%16, via two tr16 reads of 4 K rows each.
template <int RB>
__device__ __forceinline__ v4i frag_mn_bf16(const char* tile, int n0, int kk) {
    const int lane = threadIdx.x & 63, g = lane >> 4, s = lane & 15;
    v2i part[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int k = 32 * kk + 8 * g + 4 * j + (s >> 2);
        int cb = 2 * n0 + 8 * (s & 3);   // column byte
        int c = cb >> 4;
        part[j] = lds_read_tr16(tile + k * RB + ((c ^ swz_mn<2, RB>(k)) << 4) + (cb & 15));
    }
    return v4i{part[0].x, part[0].y, part[1].x, part[1].y};
}

// ---------------------------------------------------------------- work items

// K-grouped work item of one expert -> (i tile, j tile) of its dW.  Items come
// in groups of up to 4 i tiles; within a group the j tile varies slowest.  (The
// contiguous GEMM and the expert MLP use item_to_list_tiles.)
__device__ __forceinline__ void item_to_tiles(int item, int n_rt, int n_ct, int& rt, int& ct) {
    const int GM = 4;
    int per_group = GM * n_ct;
    int g = item / per_group, r = item - g * per_group;
    int gm = min(GM, n_rt - g * GM);
    ct = r / gm;
    rt = g * GM + (r - ct * gm);
}

// ---------------------------------------------------------------- contiguous / masked

// Tile configuration for the contiguous and masked kernels: 512 threads as
// WAVES_M x WAVES_N waves, each owning a WTM x WTN block of the BM x BN tile.
// A stage holds one K step (128 bytes of K per row) of both operand tiles and,
// for fp8, that step's scales: [activations | weights | scales].  The ring has
// as many stages as fit in the 160 KB of LDS, up to four: loads run
// STAGES - 1 steps ahead of the MFMAs.
template <bool FP8_, int BM_, int BN_, int WAVES_M_, int WAVES_N_, int OCC_ = 1, bool E8M0_ = false,
          bool W4_ = false>
struct GCfg {
    static constexpr bool FP8 = FP8_;
    // fp8 block scales as E8M0 exponent bytes, applied by the MFMA itself
    // (V_MFMA_SCALE_F32_16X16X128_F8F6F4) instead of promoted on the VALU
    static constexpr bool E8M0 = E8M0_;
    // weights as packed E2M1 (fp4), K-contiguous: a K step's weight row is
    // 64 bytes; the MFMA takes them as its fp4 operand
    static constexpr bool W4 = W4_;
    static constexpr int WROW = W4 ? 64 : 128;         // weight bytes per row per K step
    static constexpr int OCC = OCC_;                   // workgroups per CU the LDS ring leaves room for
    static constexpr int ESZ = FP8 ? 1 : 2;            // bytes per element
    static constexpr int KSTEP = 128 / ESZ;            // K elements per step
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int MB = WTM / 16, NB = WTN / 16;
    static constexpr int A_BYTES = BM * 128, B_BYTES = BN * WROW;
    // fp8 scales of the step: one per tile row (activations), then 256 bytes of
    // weight-block scales.  fp32: BM floats, then 64 float slots (BN / 128 of
    // them used).  E8M0: the tile's rows' bytes from a 4-byte-aligned start
    // (BM + 3 bytes in two 256-byte halves), then the N / 128 bytes of the
    // step's weight-scale row.
    static constexpr int SA_BYTES = FP8 ? (E8M0 ? 512 : BM * 4) : 0;
    static constexpr int S_BYTES = FP8 ? SA_BYTES + 256 : 0;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int STAGES =
        (160 * 1024 / OCC) / STAGE_BYTES < 4 ? (160 * 1024 / OCC) / STAGE_BYTES : 4;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_OPS = A_BYTES / 16 / THREADS;   // 16-byte DMAs per thread per step
    static constexpr int B_OPS = B_BYTES / 16 / THREADS;
    static constexpr int S_OPS = FP8 ? 1 : 0;             // one 4-byte scale DMA
    static constexpr int OPS = A_OPS + B_OPS + S_OPS;
    static_assert(WAVES == 8, "512-thread tiles");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0 && NB % 2 == 0, "wave tile");
    static_assert(A_BYTES % (16 * THREADS) == 0 && B_BYTES % (16 * THREADS) == 0, "stage split");
    static_assert(!FP8 || (BM >= 64 && BM / 64 < WAVES), "one activation-scale DMA per 64 rows, one wave left for weight scales");
    static_assert(!E8M0 || (FP8 && WAVES >= 3), "E8M0: two waves load activation-scale bytes, the others weight-scale bytes");
    static_assert(!W4 || E8M0, "fp4 weights come with E8M0 scales");
    static_assert(!FP8 || 128 % WTN == 0 || WTN % 128 == 0, "fp8 weight scale blocks");
    static_assert(STAGES >= 2 && LDS_BYTES * OCC <= 160 * 1024, "LDS budget");
};

// Contiguous: 256-column tiles, every wave tile 64 rows tall.
template <bool FP8, bool E8 = false, bool W4 = false> using Contig256 = GCfg<FP8, 256, 256, 4, 2, 1, E8, W4>;
template <bool FP8, bool E8 = false, bool W4 = false> using Contig128 = GCfg<FP8, 128, 256, 2, 4, 1, E8, W4>;
template <bool FP8, bool E8 = false, bool W4 = false> using Contig64 = GCfg<FP8, 64, 256, 1, 8, 1, E8, W4>;

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// SiLU in fp32: x * sigmoid(x) = x / (1 + e^-x); e^-x overflowing to inf for
// very negative x gives -0, the limit.
__device__ __forceinline__ float silu(float x) { return x / (1.f + expf(-x)); }

// OCP e4m3 (bias 7) code of x, |x| <= 448, round to nearest even, subnormals
// included.  Below 2^-6 the e4m3 values are multiples of 2^-9: the code is
// rint(|x| * 512) (exact scaling, rint rounds half to even; 8 is the smallest
// normal, code 0x08).  Above, the fp32 mantissa is rounded to 3 bits, nearest
// even, a carry moving into the exponent; 448 = 1.75 * 2^8 is code 0x7E.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.f);
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    return sign | ((((b >> 23) - 120u) << 3) | ((b >> 20) & 7u));
}

// One output tile of the contiguous or masked layout.
//
// Per K step every wave, in one instruction stream, reads its activation
// fragments (MB x 16 rows) and the step's scales at the start, then walks its
// NB weight blocks of 16 columns: each block's fragments are read one block
// ahead, its MFMAs issued, and (fp8) its partials promoted into the fp32
// accumulators with acc += p * a_scale[row] * b_scale[block].  Right after the
// first block's MFMAs the wave issues its share of the DMAs of step
// ks + STAGES - 1 into the stage step ks - 1 used.  One vmcnt wait plus one
// barrier per step publishes the stage of step ks + 1.
// The wave runs at raised priority (s_setprio) from the barrier to the end of
// its MFMAs, so a SIMD's two waves drain their MFMA work ahead of the barrier.
// WNT: the weight panel is read by this tile only, so its loads stream
// (non-temporal); see load16_to_lds_cp.
template <class C, bool B_KN, bool WNT = false>
struct TileGemm {
    static constexpr int WCP = WNT ? CP_NT : CP_DEFAULT;
    static constexpr int NSB = C::WTN >= 128 ? C::WTN / 128 : 1;   // weight-scale blocks per wave tile
    static constexpr int HSEG = C::WTN / 2;                        // weight rows per wave column half
    static_assert(B_KN || C::W4 || (C::B_OPS % 2 == 0 && (C::THREADS / 8) % HSEG == 0 && HSEG % 16 == 0),
                  "weight DMA row mapping");
    v4f acc[C::NB][C::MB];

    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    uint32_t a_row_bytes, b_row_bytes, b_col_byte;
    uint32_t b_step_bytes;     // K-contiguous weights: bytes between one K step's rows and the next's
    // fp32 activation scales: byte stride between tile rows and between K steps
    // ([rows, K/128]: K/128 * 4 and 4; [K/128, rows_total]: 4 and rows_total * 4)
    uint32_t sa_row_bytes, sa_step_bytes;
    uint32_t sb_col_byte;      // byte offset of this column tile's first weight-scale block in a K row
    uint32_t sb_row_bytes;     // weight-scale bytes per K step (N / 128 floats)
    int wm, wn, r16;
    // scale DMA of this wave, fixed for the whole tile so that a K step has no
    // branches: resource rss, voffset ss_voff + ks * ss_step, LDS slot ss_dst
    __amdgpu_buffer_rsrc_t rss;
    uint32_t ss_voff, ss_step, ss_dst;
    // E8M0: byte of tile row 0 inside the activation-scale slot (the slot starts
    // at the 4-byte boundary at or below the tile's first row), and the first
    // weight-scale byte of this column tile in the step's scale row
    int sa_shift, sb_col;
    uint32_t sa_step_e8;     // bytes per K-block row of the activation scales (rows_total)

    __device__ __forceinline__ void setup_roles() {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
        if constexpr (C::E8M0) {
            // waves 0-1: the activation-scale bytes (4 per lane, 512 bytes from the
            // aligned start); the others: the step's weight-scale row, N / 128 bytes
            // in the first N / 512 lanes (the rest point past the buffer and read zero)
            const bool act = wave < 2;
            rss = act ? rsa : rsb;
            ss_voff = act ? (wave * 64 + lane) * 4u : (lane * 4 < (int)sb_row_bytes ? lane * 4u : 0x80000000u);
            ss_step = act ? sa_step_e8 : sb_row_bytes;
            ss_dst = C::A_BYTES + C::B_BYTES + (act ? wave * 256 : C::SA_BYTES);
        } else if constexpr (C::FP8) {
            // waves below BM/64: one 4-byte activation scale per tile row (the
            // step's scales of the tile are one contiguous run when stored
            // [K/128, rows_total], one cache line per row otherwise); the other
            // waves: the weight-block scales of this column tile (all write the same
            // values to the same slots).  The weight-scale K row sits in voffset, so
            // the range check clamps lanes past the expert's scales.
            const bool act = wave < C::BM / 64;
            rss = act ? rsa : rsb;
            ss_voff = act ? (wave * 64 + lane) * sa_row_bytes : sb_col_byte + lane * 4;
            ss_step = act ? sa_step_bytes : sb_row_bytes;
            ss_dst = C::A_BYTES + C::B_BYTES + (act ? wave * 256 : C::SA_BYTES);
        }
    }

    // ---- the DMAs of one stage
    // activation rows r0 + 64 J; swz_k(r0 + 64 j) == swz_k(r0); the row offset stays
    // in voffset (range-checked: rows past rows_valid read as zero)
    template <int J>
    __device__ __forceinline__ void issue_a(char* __restrict__ stage, int ks) const {
        const int tid = threadIdx.x, wave = tid >> 6;
        const int r = (tid >> 3) + J * (C::THREADS / 8);
        load16_to_lds_so(ra, r * a_row_bytes + ((((tid & 7) ^ swz_k<C::ESZ>(r))) << 4), ks * 128,
                         stage + (J * C::THREADS + wave * 64) * 16);
    }

    // weight DMA J of step ks.  K-contiguous weights: DMA J covers column half
    // h = J % 2 of WAVES_N wave columns ((THREADS / 8) / HSEG of them per DMA);
    // each wave writes 8 consecutive rows.
    template <int J>
    __device__ __forceinline__ void issue_w(char* __restrict__ stage, int ks) const {
        const int tid = threadIdx.x, wave = tid >> 6;
        char* base = stage + C::A_BYTES;
        if constexpr (C::W4) {
            // 64-byte rows, four lanes per row: DMA J fills rows 16 (J * WAVES + wave)
            // and the 15 after it; the K step rides in soffset
            static_assert(!B_KN, "fp4 weights are K-contiguous");
            const int f = J * C::THREADS + tid;
            const int row = f >> 2;
            load16_to_lds_cp<WCP>(rb, row * b_row_bytes + (((f & 3) ^ swz_w4(row)) << 4), ks * b_step_bytes,
                             base + (J * C::THREADS + wave * 64) * 16);
        } else if constexpr (B_KN) {
            constexpr int RB = C::BN * C::ESZ, CPR = RB / 16, RPO = C::THREADS / CPR;
            const int r0 = tid / CPR;
            const int c = (tid % CPR) ^ swz_mn<C::ESZ, RB>(r0 + J * RPO);
            load16_to_lds_cp<WCP>(rb, r0 * b_row_bytes + b_col_byte + c * 16, (ks * C::KSTEP + J * RPO) * b_row_bytes,
                             base + (J * C::THREADS + wave * 64) * 16);
        } else {
            constexpr int h = J & 1, q = J >> 1, SPO = (C::THREADS / 8) / HSEG;
            auto row_of = [](int lr) { return (q * SPO + lr / HSEG) * C::WTN + h * HSEG + lr % HSEG; };
            const int row = row_of(tid >> 3);
            load16_to_lds_cp<WCP>(rb, row * b_row_bytes + (((tid & 7) ^ swz_k<C::ESZ>(row)) << 4), ks * b_step_bytes,
                             base + row_of(wave * 8) * 128);
        }
    }

    __device__ __forceinline__ void issue_s(char* __restrict__ stage, int ks) const {
        if constexpr (C::E8M0)
            // the K-block row goes in soffset, the lane's bytes in voffset (lanes with
            // nothing to load are parked past the buffer and read zero)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rss, (MOEGG_LDS void*)(stage + ss_dst), 4, ss_voff,
                                                     ks * ss_step, 0, 0);
        else if constexpr (C::FP8)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rss, (MOEGG_LDS void*)(stage + ss_dst), 4,
                                                     ss_voff + ks * ss_step, 0, 0, 0);
    }

    // all DMAs of step ks into `stage`
    __device__ __forceinline__ void issue_all(char* __restrict__ stage, int ks) const {
        static_for<0, C::A_OPS>([&](auto J) { issue_a<decltype(J)::value>(stage, ks); });
        static_for<0, C::B_OPS>([&](auto J) { issue_w<decltype(J)::value>(stage, ks); });
        issue_s(stage, ks);
    }

    __device__ __forceinline__ static void promote(v4f& a, const v4f q, float s) {
        a.x = __builtin_fmaf(q.x, s, a.x);
        a.y = __builtin_fmaf(q.y, s, a.y);
        a.z = __builtin_fmaf(q.z, s, a.z);
        a.w = __builtin_fmaf(q.w, s, a.w);
    }

    __device__ __forceinline__ static void barrier() {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    }

    // One K step for a wave with MBA active 16-row blocks.
    // One K step: reads stage `ta`, issues the DMAs of step `next` into stage `wr`.
    // The two are different stages; saying so (__restrict__) lets the compiler
    // see that the transpose reads do not depend on the DMAs in flight.
    template <int MBA>
    __device__ __forceinline__ void step(const char* __restrict__ ta, char* __restrict__ wr, int next) {
        const char* tb = ta + C::A_BYTES;
        if constexpr (MBA == 0) {
            issue_all(wr, next);
        } else if constexpr (C::E8M0) {
            // scales go to the MFMA: scale_a (weights, the A operand) is the byte of
            // the 128-column block, the same in every lane; scale_b (activations)
            // is each lane's row byte.  The MFMA accumulates straight into acc.
            const MOEGG_LDS unsigned char* sab = (const MOEGG_LDS unsigned char*)(tb + C::B_BYTES) + sa_shift;
            const MOEGG_LDS unsigned char* sbb = (const MOEGG_LDS unsigned char*)(tb + C::B_BYTES + C::SA_BYTES) + sb_col;
            auto fragb = [&](int i) -> v8i {
                const int n0 = wn * C::WTN + i * 16;
                if constexpr (C::W4) return frag_k_fp4(tb, n0 + r16);
                else if constexpr (B_KN) return frag_mn_fp8<C::BN>(tb, n0);
                else return frag_k_fp8(tb, n0 + r16);
            };
            // operand formats: 4 = E2M1 (fp4) weights, 0 = e4m3
            constexpr int FMT_W = C::W4 ? 4 : 0;
            v8i xb[2];
            xb[0] = fragb(0);
            v8i ya[MBA];
            int sbj[MBA];
#pragma unroll
            for (int j = 0; j < MBA; ++j) {
                if constexpr (C::W4) ya[j] = frag_k_fp8_mfma_order(ta, wm * C::WTM + j * 16 + r16);
                else ya[j] = frag_k_fp8(ta, wm * C::WTM + j * 16 + r16);
            }
#pragma unroll
            for (int j = 0; j < MBA; ++j) sbj[j] = sab[wm * C::WTM + j * 16 + r16];
            int sai[NSB];
#pragma unroll
            for (int b = 0; b < NSB; ++b) sai[b] = sbb[(wn * C::WTN) / 128 + b];
            static_for<0, C::NB>([&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (i + 1 < C::NB) xb[(i + 1) & 1] = fragb(i + 1);
                constexpr int sb = NSB > 1 ? i * 16 / 128 : 0;
#pragma unroll
                for (int j = 0; j < MBA; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xb[i & 1], ya[j], acc[i][j], FMT_W,
                                                                                 0, 0, sai[sb], 0, sbj[j]);
                if constexpr (i == 0) issue_all(wr, next);
                __builtin_amdgcn_sched_barrier(0);
            });
        } else if constexpr (C::FP8) {
            const float* ts = (const float*)(tb + C::B_BYTES);
            const float* tsb = (const float*)(tb + C::B_BYTES + C::SA_BYTES) + wn * C::WTN / 128;
            auto fragb = [&](int i) -> v8i {
                const int n0 = wn * C::WTN + i * 16;
                if constexpr (B_KN) return frag_mn_fp8<C::BN>(tb, n0);
                else return frag_k_fp8(tb, n0 + r16);
            };
            // LDS reads in the order the first MFMAs consume them: weight block 0,
            // activation blocks, then the scales
            v8i xb[2];
            xb[0] = fragb(0);
            v8i ya[MBA];
#pragma unroll
            for (int j = 0; j < MBA; ++j) ya[j] = frag_k_fp8(ta, wm * C::WTM + j * 16 + r16);
            float bsc[NSB], s[NSB][MBA];
#pragma unroll
            for (int b = 0; b < NSB; ++b) bsc[b] = tsb[b];
#pragma unroll
            for (int j = 0; j < MBA; ++j) {
                const float as = ts[wm * C::WTM + j * 16 + r16];
#pragma unroll
                for (int b = 0; b < NSB; ++b) s[b][j] = as * bsc[b];
            }
            // Software-pipelined promotion: block i's MFMAs are interleaved with the
            // promotion of block i - 1's partials, which finished a block earlier, so
            // the four FMAs that follow each MFMA never wait on a result and run on
            // the VALU while the MFMA occupies the matrix pipe.  Each accumulator
            // still receives the same products in the same order.
            v4f p[2][MBA];
            static_for<0, C::NB + 1>([&](auto I) {
                constexpr int i = decltype(I)::value;
                constexpr int ip = i - 1;                               // block promoted now
                constexpr int sbp = ip >= 0 && NSB > 1 ? ip * 16 / 128 : 0;
                if constexpr (i + 1 < C::NB) xb[(i + 1) & 1] = fragb(i + 1);
#pragma unroll
                for (int j = 0; j < MBA; ++j) {
                    if constexpr (i < C::NB) p[i & 1][j] = mfma_fp8(xb[i & 1], ya[j], v4f{0.f, 0.f, 0.f, 0.f});
                    if constexpr (ip >= 0) promote(acc[ip][j], p[ip & 1][j], s[sbp][j]);
                }
                if constexpr (i == 0) issue_all(wr, next);
                if constexpr (i > 0 && i < C::NB) {
#pragma unroll
                    for (int j = 0; j < MBA; ++j) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);     // then four VALU ops
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            // both K halves of the step's activation fragments first, then the weight
            // blocks column half by column half
            v4i ya[2][MBA];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int j = 0; j < MBA; ++j) ya[kk][j] = frag_k_bf16(ta, wm * C::WTM + j * 16 + r16, kk);
            auto fragb = [&](int i, int kk) -> v4i {
                const int n0 = wn * C::WTN + i * 16;
                if constexpr (B_KN) return frag_mn_bf16<C::BN * 2>(tb, n0, kk);
                else return frag_k_bf16(tb, n0 + r16, kk);
            };
            v4i xb[2];
            xb[0] = fragb(0, 0);
            static_for<0, 2 * C::NB>([&](auto U) {
                constexpr int u = decltype(U)::value, i = u >> 1, kk = u & 1;
                if constexpr (u + 1 < 2 * C::NB) xb[(u + 1) & 1] = fragb((u + 1) >> 1, (u + 1) & 1);
#pragma unroll
                for (int j = 0; j < MBA; ++j) acc[i][j] = mfma_bf16(xb[u & 1], ya[kk][j], acc[i][j]);
                if constexpr (u == 0) issue_all(wr, next);
                __builtin_amdgcn_sched_barrier(0);
            });
        }
    }

    // Every step issues exactly OPS DMAs per wave (steps past the last are
    // clamped to the last one and land in a free stage), so an in-order vmcnt
    // wait with a fixed allowance -- the STAGES - 2 newest batches -- publishes
    // the stage of the next step.
    template <int MBA>
    __device__ __forceinline__ void kloop(char* lds, int nks) {
        constexpr int S = C::STAGES;
#pragma unroll
        for (int s = 0; s < S - 1; ++s) issue_all(lds + s * C::STAGE_BYTES, min(s, nks - 1));
        wait_vmcnt<(S - 2) * C::OPS>();
        barrier();
        int cur = 0, free = S - 1;
        for (int ks = 0; ks < nks; ++ks) {
            __builtin_amdgcn_s_setprio(1);
            step<MBA>(lds + cur * C::STAGE_BYTES, lds + free * C::STAGE_BYTES, min(ks + S - 1, nks - 1));
            __builtin_amdgcn_s_setprio(0);
            wait_vmcnt<(S - 2) * C::OPS>();   // this wave's DMAs of step ks + 1 landed
            barrier();
            free = cur;
            cur = cur + 1 == S ? 0 : cur + 1;
        }
        // no LDS DMA may still be in flight when the wave moves on or exits
        wait_vmcnt<0>();
    }

    template <int M>
    __device__ __forceinline__ void dispatch(char* lds, int mba, int nks) {
        if constexpr (M < 0) {
            return;
        } else {
            if (mba == M) kloop<M>(lds, nks);
            else dispatch<M - 1>(lds, mba, nks);
        }
    }

    __device__ __forceinline__ void run(char* lds, int nks, int rows_valid) {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        wm = wave / C::WAVES_N;
        wn = wave % C::WAVES_N;
        r16 = lane & 15;
#pragma unroll
        for (int i = 0; i < C::NB; ++i)
#pragma unroll
            for (int j = 0; j < C::MB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        setup_roles();
        // active 16-row blocks of this wave; wave-uniform, so the loop has no divergence
        const int mba = __builtin_amdgcn_readfirstlane(min(C::MB, max(0, (rows_valid - wm * C::WTM + 15) >> 4)));
        dispatch<C::MB>(lds, mba, nks);
    }

    // ---- epilogues staged through LDS
    // An output tile of BM rows of RB bytes is written to LDS first, 16-byte
    // chunks XOR-swizzled by the row (row & 15, or & 7 for 8-chunk rows), then
    // stored as whole rows, 16 bytes per lane, so each store instruction writes
    // THREADS * 16 consecutive-row bytes instead of a few bytes of each of 16
    // rows.  Byte b of tile row r sits at lds_off<RB>(r, b).
    template <int RB>
    __device__ __forceinline__ static int lds_off(int row, int byte) {
        constexpr int CPR = RB / 16;
        static_assert(CPR >= 8 && C::THREADS % CPR == 0, "row swizzle");
        return row * RB + ((((byte >> 4) ^ (row & (CPR >= 16 ? 15 : 7)))) << 4) + (byte & 15);
    }

    // Stores rows < rows_valid of the staged tile (after a barrier that
    // published it); output rows are row_bytes apart in rc.  Stores past the
    // valid rows fall outside rc and are dropped; whole passes past them are
    // skipped.
    template <int RB>
    __device__ __forceinline__ static void store_staged(const char* lds, __amdgpu_buffer_rsrc_t rc,
                                                        uint32_t row_bytes, int rows_valid) {
        constexpr int CPR = RB / 16, ROWS_PER_PASS = C::THREADS / CPR;
        static_assert(C::BM * RB <= C::LDS_BYTES, "the staged tile fits in the ring");
        const int c = threadIdx.x % CPR;
#pragma unroll 4
        for (int r0 = 0; r0 < C::BM; r0 += ROWS_PER_PASS) {
            if (r0 >= rows_valid) break;
            const int row = r0 + threadIdx.x / CPR;
            const v4i v = lds_read_b128(lds + lds_off<RB>(row, c * 16));
            __builtin_amdgcn_raw_buffer_store_b128(v, rc, row * row_bytes + c * 16, 0, 0);
        }
    }

    // bf16 epilogue: rows < rows_valid of the tile; C rows are row_bytes apart.
    // The first barrier makes the ring free: every wave's last DMAs have landed
    // (each waited for its own before it).
    __device__ __forceinline__ void store_bf16(__amdgpu_buffer_rsrc_t rc, uint32_t row_bytes, int rows_valid,
                                               char* lds) {
        constexpr int RB = C::BN * 2;
        const int g = (threadIdx.x & 63) >> 4;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < C::MB; ++j) {
            const int row = wm * C::WTM + j * 16 + r16;
#pragma unroll
            for (int i = 0; i < C::NB; ++i) {
                const int col = wn * C::WTN + i * 16 + 4 * g;
                v2i d;
                d.x = (int)pack_bf16x2(acc[i][j].x, acc[i][j].y);
                d.y = (int)pack_bf16x2(acc[i][j].z, acc[i][j].w);
                *(MOEGG_LDS v2i*)(lds + lds_off<RB>(row, col * 2)) = d;
            }
        }
        __syncthreads();
        store_staged<RB>(lds, rc, row_bytes, rows_valid);
    }

    // SwiGLU epilogue: the tile's columns come in groups of 32, gate columns
    // then the matching up columns, so blocks 2i and 2i + 1 of a wave hold the
    // gate and up values of the same 16 outputs in the same lanes.  Writes
    // silu(gate) * up as bf16: 4 consecutive outputs per lane, rows <
    // rows_valid, output row_bytes apart, BN / 2 outputs per tile.
    __device__ __forceinline__ void store_swiglu(__amdgpu_buffer_rsrc_t rc, uint32_t row_bytes, int rows_valid,
                                                 char* lds) {
        static_assert(C::NB % 2 == 0, "gate/up block pairs");
        constexpr int RB = C::BN;                        // BN / 2 bf16 outputs per row
        const int g = (threadIdx.x & 63) >> 4;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < C::MB; ++j) {
            const int row = wm * C::WTM + j * 16 + r16;
#pragma unroll
            for (int ip = 0; ip < C::NB / 2; ++ip) {
                const v4f gt = acc[2 * ip][j], up = acc[2 * ip + 1][j];
                const int col = wn * C::WTN / 2 + ip * 16 + 4 * g;
                v2i d;
                d.x = (int)pack_bf16x2(silu(gt.x) * up.x, silu(gt.y) * up.y);
                d.y = (int)pack_bf16x2(silu(gt.z) * up.z, silu(gt.w) * up.w);
                *(MOEGG_LDS v2i*)(lds + lds_off<RB>(row, col * 2)) = d;
            }
        }
        __syncthreads();
        store_staged<RB>(lds, rc, row_bytes, rows_valid);
    }

    // SwiGLU epilogue with H quantized for an e4m3 down projection: the tile's
    // BN / 2 = 128 outputs of a row form one 1x128 group.  Its amax is reduced
    // over the lane's 4 x NB / 2 values, the four lane groups holding the row
    // (lane shuffles) and the WAVES_N wave columns (through LDS, which no stage
    // uses any more); scale = amax / 448 (1 when amax = 0); code = e4m3(h /
    // scale), clamped to +-448, round to nearest even (e4m3_code).  The codes are
    // staged in LDS behind the amax exchange and stored to rh as whole rows; the
    // scale goes to rs[row, group].
    __device__ __forceinline__ void store_swiglu_e4m3(__amdgpu_buffer_rsrc_t rh, uint32_t row_bytes,
                                                      __amdgpu_buffer_rsrc_t rs, uint32_t s_row_bytes,
                                                      uint32_t s_group_bytes, int group,
                                                      char* lds, int rows_valid) {
        static_assert(C::NB % 2 == 0 && C::BN == 256, "one 128-wide group per tile row");
        const int lane = threadIdx.x & 63, g = lane >> 4;
        float h[C::MB][C::NB / 2][4];
        float amax[C::MB];
#pragma unroll
        for (int j = 0; j < C::MB; ++j) {
            amax[j] = 0.f;
#pragma unroll
            for (int ip = 0; ip < C::NB / 2; ++ip) {
                const v4f gt = acc[2 * ip][j], up = acc[2 * ip + 1][j];
                h[j][ip][0] = silu(gt.x) * up.x;
                h[j][ip][1] = silu(gt.y) * up.y;
                h[j][ip][2] = silu(gt.z) * up.z;
                h[j][ip][3] = silu(gt.w) * up.w;
#pragma unroll
                for (int t = 0; t < 4; ++t) amax[j] = fmaxf(amax[j], fabsf(h[j][ip][t]));
            }
            amax[j] = fmaxf(amax[j], __shfl_xor(amax[j], 16, 64));
            amax[j] = fmaxf(amax[j], __shfl_xor(amax[j], 32, 64));
        }
        // every wave's DMAs have landed once all waves pass this barrier
        __syncthreads();
        float* red = (float*)lds;                             // [WAVES_N][BM]
        // the staged codes [BM][BN / 2] follow the amax exchange
        constexpr int RED_BYTES = 4096;
        static_assert(C::WAVES_N * C::BM * 4 <= RED_BYTES && RED_BYTES + C::BM * C::BN / 2 <= C::LDS_BYTES,
                      "epilogue LDS");
        char* codes = lds + RED_BYTES;
        if (g == 0) {
#pragma unroll
            for (int j = 0; j < C::MB; ++j) red[wn * C::BM + wm * C::WTM + j * 16 + r16] = amax[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < C::MB; ++j) {
            const int row = wm * C::WTM + j * 16 + r16;
            float m = 0.f;
#pragma unroll
            for (int w = 0; w < C::WAVES_N; ++w) m = fmaxf(m, red[w * C::BM + row]);
            const float scale = m > 0.f ? m / 448.f : 1.f;
            // codes of every row go to the staged tile (rows past the valid ones
            // are never stored; the clamp turns a NaN into -448 first)
#pragma unroll
            for (int ip = 0; ip < C::NB / 2; ++ip) {
                uint32_t v = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    v |= e4m3_code(fminf(fmaxf(h[j][ip][t] / scale, -448.f), 448.f)) << (8 * t);
                const int col = wn * C::WTN / 2 + ip * 16 + 4 * g;
                *(MOEGG_LDS uint32_t*)(codes + lds_off<C::BN / 2>(row, col)) = v;
            }
            if (row < rows_valid && wn == 0 && g == 0)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, scale), rs,
                                                      row * s_row_bytes + group * s_group_bytes, 0, 0);
        }
        __syncthreads();
        store_staged<C::BN / 2>(codes, rh, row_bytes, rows_valid);
    }
};

// One output tile: rows [row_start, row_start + rows_valid) of expert e's
// segment, column tile ct.
template <class C, bool B_KN, int SWIGLU = 0, bool WNT = false>
__device__ __forceinline__ void contig_tile(const ContigArgs& p, char* lds, int e, int row_start, int rows_valid,
                                            int ct) {
    if constexpr (C::W4 && WNT) {
        // fp4 weights stream only in panels: stored [G, N, K/2], a K step reads half of each
        // 128-byte line, and a line loaded non-temporally is gone before the next step reads
        // its other half
        if (!p.b_panel) {
            contig_tile<C, B_KN, SWIGLU, false>(p, lds, e, row_start, rows_valid, ct);
            return;
        }
    }
    const int n0 = ct * C::BN;
    const int KB = p.K / 128;
    TileGemm<C, B_KN, WNT> tg;
    tg.a_row_bytes = (uint32_t)p.K * C::ESZ;
    tg.ra = make_rsrc((const char*)p.A + (size_t)row_start * tg.a_row_bytes, (uint32_t)rows_valid * tg.a_row_bytes);
    const size_t b_expert_bytes = C::W4 ? (size_t)p.K * p.N / 2 : (size_t)p.K * p.N * C::ESZ;
    const char* b_base = (const char*)p.B + (size_t)e * b_expert_bytes;
    if constexpr (C::W4) {
        if (p.b_panel) {
            // packed E2M1 [G, N / BN, K / 128, BN, 64]: one K step of the column tile's BN rows back to
            // back, so a step reads whole 128-byte lines
            tg.rb = make_rsrc(b_base + (size_t)ct * C::BN * (p.K / 2), (uint32_t)C::BN * (p.K / 2));
            tg.b_row_bytes = C::WROW;
            tg.b_step_bytes = (uint32_t)C::BN * C::WROW;
        } else {
            // packed E2M1 [G, N, K/2]: this column tile's BN rows of K/2 bytes; a step reads
            // 64 bytes of each, half a line
            tg.b_row_bytes = (uint32_t)p.K / 2;
            tg.rb = make_rsrc(b_base + (size_t)n0 * tg.b_row_bytes, (uint32_t)C::BN * tg.b_row_bytes);
            tg.b_step_bytes = C::WROW;
        }
        tg.b_col_byte = 0;
    } else if constexpr (B_KN) {
        if (p.b_panel) {
            // [G, N / BN, K, BN]: this column tile's panel, K rows of BN columns back to back
            tg.rb = make_rsrc(b_base + (size_t)ct * p.K * C::BN * C::ESZ, (uint32_t)p.K * C::BN * C::ESZ);
            tg.b_row_bytes = (uint32_t)C::BN * C::ESZ;
            tg.b_col_byte = 0;
        } else {
            tg.rb = make_rsrc(b_base, (uint32_t)b_expert_bytes);
            tg.b_row_bytes = (uint32_t)p.N * C::ESZ;
            tg.b_col_byte = (uint32_t)n0 * C::ESZ;
        }
    } else {
        tg.rb = make_rsrc(b_base + (size_t)n0 * p.K * C::ESZ, (uint32_t)C::BN * p.K * C::ESZ);
        if (p.b_panel) {
            // [G, N / BN, K / KSTEP, BN, KSTEP]: one K step of the column tile's BN rows back to back
            tg.b_row_bytes = 128;
            tg.b_step_bytes = (uint32_t)C::BN * 128;
        } else {
            tg.b_row_bytes = (uint32_t)p.K * C::ESZ;
            tg.b_step_bytes = 128;
        }
        tg.b_col_byte = 0;
    }
    tg.rsa = tg.rb;
    tg.rsb = tg.rb;
    tg.sa_row_bytes = p.a_scale_km ? 4u : (uint32_t)KB * 4;
    tg.sa_step_bytes = p.a_scale_km ? (uint32_t)p.rows_total * 4 : 4u;
    tg.sb_row_bytes = (uint32_t)(p.N / 128) * 4;
    tg.sb_col_byte = (uint32_t)(n0 / 128) * 4;
    if constexpr (C::E8M0) {
        // activation-scale bytes [K/128, rows_total]: the step's row of bytes from
        // the 4-byte boundary at or below the tile's first row (the step's row
        // offset rides in soffset, which the range check counts too, so the
        // resource spans every K-block row); rows_total % 4 == 0, so no dword
        // crosses the end of the array
        const int a0 = row_start & ~3;
        tg.sa_shift = row_start - a0;
        tg.sa_step_e8 = (uint32_t)p.rows_total;
        tg.rsa = make_rsrc((const unsigned char*)p.A_scale + a0, (uint32_t)((int64_t)KB * p.rows_total - a0));
        // weight-scale bytes [G, K/128, N/128]: this expert's block, one row per step
        tg.sb_row_bytes = (uint32_t)(p.N / 128);
        tg.sb_col = n0 / 128;
        tg.rsb = make_rsrc((const unsigned char*)p.B_scale + (size_t)e * KB * (p.N / 128), (uint32_t)KB * (p.N / 128));
    } else if constexpr (C::FP8) {
        // rows past rows_valid: zeros from the range check ([rows, K/128]), or the
        // neighbouring rows' scales ([K/128, rows_total]), which only ever meet
        // those rows' zero activations and are never stored
        tg.rsa = p.a_scale_km
                     ? make_rsrc((const float*)p.A_scale + row_start, (uint32_t)(((int64_t)KB * p.rows_total - row_start) * 4))
                     : make_rsrc((const float*)p.A_scale + (size_t)row_start * KB, (uint32_t)rows_valid * KB * 4);
        // this expert's weight scales [K/128, N/128]; slots past the row read as zero
        tg.rsb = make_rsrc((const float*)p.B_scale + (size_t)e * KB * (p.N / 128), (uint32_t)KB * tg.sb_row_bytes);
    }
    tg.run(lds, p.K / C::KSTEP, rows_valid);
    if constexpr (SWIGLU == 2) {
        // output H e4m3 [rows_total, N / 2] and its scales [rows_total, N / 256]: the tile's
        // BN / 2 = 128 outputs per row are one scale group (group ct)
        const uint32_t h_row_bytes = (uint32_t)p.N / 2;
        // [rows_total, N / 256], or [N / 256, rows_total] with a_scale_km
        const uint32_t s_row_bytes = p.a_scale_km ? 4u : (uint32_t)(p.N / 256) * 4;
        const uint32_t s_group_bytes = p.a_scale_km ? (uint32_t)p.rows_total * 4 : 4u;
        auto rh = make_rsrc((char*)p.C + (size_t)row_start * h_row_bytes + (size_t)ct * (C::BN / 2),
                            (uint32_t)(rows_valid - 1) * h_row_bytes + C::BN / 2);
        auto rs = p.a_scale_km
                      ? make_rsrc((float*)p.C_scale + row_start, (uint32_t)(((int64_t)(p.N / 256) * p.rows_total - row_start) * 4))
                      : make_rsrc((char*)p.C_scale + (size_t)row_start * s_row_bytes, (uint32_t)rows_valid * s_row_bytes);
        tg.store_swiglu_e4m3(rh, h_row_bytes, rs, s_row_bytes, s_group_bytes, ct, lds, rows_valid);
    } else if constexpr (SWIGLU == 1) {
        // output H [rows_total, N / 2]: the tile's BN interleaved columns give BN / 2 outputs
        const uint32_t h_row_bytes = (uint32_t)p.N;              // N / 2 bf16
        auto rh = make_rsrc((char*)p.C + (size_t)row_start * h_row_bytes + (size_t)n0,
                            (uint32_t)(rows_valid - 1) * h_row_bytes + C::BN);
        tg.store_swiglu(rh, h_row_bytes, rows_valid, lds);
    } else {
        const uint32_t c_row_bytes = (uint32_t)p.N * 2;
        auto rc = make_rsrc((char*)p.C + (size_t)row_start * c_row_bytes + (size_t)n0 * 2,
                            (uint32_t)(rows_valid - 1) * c_row_bytes + C::BN * 2);
        tg.store_bf16(rc, c_row_bytes, rows_valid, lds);
    }
}

// M-grouped contiguous layout, one tile height.
template <class C, bool B_KN, int SWIGLU = 0>
__global__ __launch_bounds__(C::THREADS, C::OCC) void grouped_gemm_kernel(ContigArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    const int n_ct = p.N / C::BN;
    const WsLayout L = ws_layout(p.G, 0);
    const Control* ctl = (const Control*)(p.ws + L.control);
    if (ctl->block_m != C::BM) return;       // another candidate height was chosen
    const int n_rt = ctl->n_tiles;
    const int item = block_to_item(blockIdx.x);
    if (item >= n_rt * n_ct) return;
    int rt, ct;
    item_to_list_tiles(item, n_rt, n_ct, (const moegg_tile_t*)(p.ws + L.tiles), false, rt, ct);
    const moegg_tile_t t = ((const moegg_tile_t*)(p.ws + L.tiles))[rt];
    if (t.tile == 0 && t.rows_valid < C::BM) {
        // the expert's only tile: this column's weight panel has no other reader, so it streams
        contig_tile<C, B_KN, SWIGLU, true>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
        return;
    }
    contig_tile<C, B_KN, SWIGLU>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
}

// Masked layout: one workgroup per (expert, 128-column tile).  It reads
// masked_m[e] itself, so an empty expert loads no weights and the grid depends
// only on G and N, and it walks the expert's rows in 128-row tiles, the last
// one 64 or 128 rows tall.  An expert of one tile is its weight panel's only
// reader, so the panel streams; with several, every tile loads it again.
// Two workgroups per CU (four waves per SIMD, so at most 128 VGPRs; 80 KB of
// LDS each): the loads of one overlap the start-up and epilogue of the other.
// A 256-row height would need a 48 KB stage and one workgroup per CU, which
// costs the short tiles that decode mostly runs more than it saves.
template <bool FP8, bool E8 = false, bool W4 = false> using Masked64 = GCfg<FP8, 64, 128, 2, 4, 2, E8, W4>;
template <bool FP8, bool E8 = false, bool W4 = false> using Masked128 = GCfg<FP8, 128, 128, 4, 2, 2, E8, W4>;

template <bool FP8, bool E8, bool W4, bool NT, bool B_KN>
__device__ __forceinline__ void masked_tile(const ContigArgs& p, char* lds, int e, int row_start, int rows, int ct) {
    if (rows > 64)
        contig_tile<Masked128<FP8, E8, W4>, B_KN, 0, NT>(p, lds, e, row_start, rows, ct);
    else
        contig_tile<Masked64<FP8, E8, W4>, B_KN, 0, NT>(p, lds, e, row_start, rows, ct);
}

template <bool FP8, bool B_KN, bool E8, bool W4>
__global__ __launch_bounds__(512, 4) void grouped_gemm_masked_kernel(ContigArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    const int n_ct = p.N / 128;
    const int e = blockIdx.x / n_ct, ct = blockIdx.x - e * n_ct;
    if (e >= p.G) return;
    const int m = min(max(p.counts[e], 0), p.cap);
    if (m == 0) return;
    const int row0 = e * p.cap;
    if (m <= 128) {
        masked_tile<FP8, E8, W4, true, B_KN>(p, lds, e, row0, m, ct);
        return;
    }
    const int last = (m - 1) >> 7;           // tiles before the last
#pragma unroll 1
    for (int i = 0; i < last; ++i) {
        if (i > 0) __syncthreads();         // the previous tile's LDS is free
        contig_tile<Masked128<FP8, E8, W4>, B_KN>(p, lds, e, row0 + i * 128, 128, ct);
    }
    __syncthreads();
    masked_tile<FP8, E8, W4, false, B_KN>(p, lds, e, row0 + last * 128, m - last * 128, ct);
}

// One launch for any tile height the scheduler chose (block_m = 0, the
// choice made on the device) and for per-expert heights
// (MOEGG_BLOCK_M_PER_EXPERT).  The grid is sized from host arguments for the
// longest list any height can produce (64-row tiles); each workgroup runs one
// work item with the configuration of the chosen height, or under per-expert
// heights with the smallest one that holds the tile's valid rows, and
// workgroups past the list exit after reading the control block.  (A grid
// sized for 256-row tiles with a loop over items spilled registers: the
// compiler kept tile setup of all three configurations live across the loop.)
// The per-expert list orders tiles of more than 128 valid rows first, then
// tails of 65..128 rows, then tails of 1..64 rows, so an expert's remainder
// does not pay for a 256-row tile and the 128- and 64-row configurations'
// deeper stage rings keep their loads further ahead.  Nothing here depends on
// the host knowing the height, so the call is graph-capturable.
template <bool FP8, bool B_KN, bool E8, bool W4, int SWIGLU = 0>
__global__ __launch_bounds__(512, 1) void grouped_gemm_auto_kernel(ContigArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    const int n_ct = p.N / 256;
    const WsLayout L = ws_layout(p.G, 0);
    const Control* ctl = (const Control*)(p.ws + L.control);
    const int bm = ctl->block_m;
    if (p.req_block_m != 0 && p.req_block_m != bm) return;   // asked for another height than scheduled
    const int n_rt = ctl->n_tiles;
    const moegg_tile_t* tiles = (const moegg_tile_t*)(p.ws + L.tiles);
    const int item = block_to_item(blockIdx.x);
    if (item >= n_rt * n_ct) return;
    int rt, ct;
    item_to_list_tiles(item, n_rt, n_ct, tiles, bm == MOEGG_BLOCK_M_PER_EXPERT, rt, ct);
    const moegg_tile_t t = tiles[rt];
    // A weight panel that one tile alone reads streams (non-temporal loads): the per-expert list's tails
    // (1..128 rows, run after all full tiles) and, at any height, an expert's only tile.
    const bool alone = t.tile == 0 && t.rows_valid < (bm == MOEGG_BLOCK_M_PER_EXPERT || bm == 256 ? 256 : bm);
    if (bm == MOEGG_BLOCK_M_PER_EXPERT) {
        if (t.rows_valid > 128) {
            if (alone)
                contig_tile<Contig256<FP8, E8, W4>, B_KN, SWIGLU, true>(p, lds, t.expert, t.row_start, t.rows_valid,
                                                                        ct);
            else
                contig_tile<Contig256<FP8, E8, W4>, B_KN, SWIGLU>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
        } else if (t.rows_valid > 64) {
            contig_tile<Contig128<FP8, E8, W4>, B_KN, SWIGLU, true>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
        } else {
            contig_tile<Contig64<FP8, E8, W4>, B_KN, SWIGLU, true>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
        }
    } else if (bm == 256) {
        if (alone)
            contig_tile<Contig256<FP8, E8, W4>, B_KN, SWIGLU, true>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
        else
            contig_tile<Contig256<FP8, E8, W4>, B_KN, SWIGLU>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
    } else if (bm == 128) {
        if (alone)
            contig_tile<Contig128<FP8, E8, W4>, B_KN, SWIGLU, true>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
        else
            contig_tile<Contig128<FP8, E8, W4>, B_KN, SWIGLU>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
    } else {
        if (alone)
            contig_tile<Contig64<FP8, E8, W4>, B_KN, SWIGLU, true>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
        else
            contig_tile<Contig64<FP8, E8, W4>, B_KN, SWIGLU>(p, lds, t.expert, t.row_start, t.rows_valid, ct);
    }
}

// ---------------------------------------------------------------- expert MLP, one launch

constexpr int kMlpSpinLimit = 1 << 15;      // polls (with a short sleep each) before a wait gives up

// The expert MLP (the compute half of the DeepGEMM record's Mega MoE: both
// expert GEMMs and SwiGLU in one kernel, "Arithmetic intensity") in one
// launch, so the down projection of a row tile starts as soon as its H is
// complete and the two GEMMs share one tail instead of two.  (H still goes
// through its buffer: each release writes the XCD's L2 back.)  One workgroup
// per work item, statically: the grid holds all L1 items first, then all L2
// items, each phase in the contiguous GEMM's order (runs of 32 items per XCD,
// row tiles of one expert in groups of four), so each phase shares operands
// across XCDs as the two launches of the chain do.
//   L1 item (rt, c): the SwiGLU tile writing H rows of rt, columns [128c,
//   128c + 128), and their scales; every wave waits for its stores, then one
//   thread releases (agent scope) an increment of rt's completion counter.
//   L2 item (rt, c): one thread polls rt's counter until all C1 L1 items of
//   rt have counted, acquires (agent scope: this CU's L1 holds no stale H),
//   then the tile of Y = H W2 runs.  The wait is bounded: past the poll limit
//   it sets MOEGG_FLAG_SYNC_TIMEOUT, which also ends every later wait at once,
//   and goes on (those output rows are then unspecified).
// Deadlock-free: an L2 workgroup waits only on L1 workgroups, which wait on
// nothing and all have lower indices.  Workgroups are dispatched in index
// order, so when an L2 workgroup runs every L1 workgroup has been dispatched
// and finishes.  The lone tile of an expert (its only row tile, not full)
// streams its weight panel, as in the contiguous GEMM.
__global__ __launch_bounds__(512, 1) void expert_mlp_fused_kernel(MlpArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    using C = Contig256<true>;
    const WsLayout L = ws_layout(p.l1.G, 0);
    const Control* ctl = (const Control*)(p.l1.ws + L.control);
    if (ctl->block_m != 256) return;         // needs the 256-row schedule
    const moegg_tile_t* tiles = (const moegg_tile_t*)(p.l1.ws + L.tiles);
    const int C1 = p.l1.N / 256, C2 = p.l2.N / 256;
    int phase, rt, c;
    if (!mlp_block_item((int)blockIdx.x, p.l1_blocks, ctl->n_tiles, C1, C2, tiles, phase, rt, c)) return;
    const moegg_tile_t t = tiles[rt];
    const bool alone = t.tile == 0 && t.rows_valid < C::BM;
    uint32_t* done = p.sync + rt;
    if (phase == 1) {
        if (alone)
            contig_tile<C, false, 2, true>(p.l1, lds, t.expert, t.row_start, t.rows_valid, c);
        else
            contig_tile<C, false, 2>(p.l1, lds, t.expert, t.row_start, t.rows_valid, c);
        wait_vmcnt<0>();                      // this wave's H stores are done
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        if (threadIdx.x == 0) {
            moegg_stats_t* st = (moegg_stats_t*)(const_cast<unsigned char*>(p.l1.ws) + L.stats);
            int polls = 0;
            while (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)C1) {
                if (++polls > kMlpSpinLimit ||
                    (__hip_atomic_load(&st->error_flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                     MOEGG_FLAG_SYNC_TIMEOUT)) {
                    __hip_atomic_fetch_or(&st->error_flags, MOEGG_FLAG_SYNC_TIMEOUT, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        if (alone)
            contig_tile<C, false, 0, true>(p.l2, lds, t.expert, t.row_start, t.rows_valid, c);
        else
            contig_tile<C, false, 0>(p.l2, lds, t.expert, t.row_start, t.rows_valid, c);
    }
}

// ---------------------------------------------------------------- K-grouped


// dW[e, i, j] = sum over expert e's rows t of X[t, i] * dY[t, j].
// Both operands are M/N-contiguous: the dY tile is the MFMA A operand (so each
// lane holds 4 consecutive j), the X tile the MFMA B operand.
// fp8 (C::FP8): X and dY are e4m3 codes; a stage is one 128-row scale group of
// the expert's segment (groups restart at its first row), and each group's
// partial sum is promoted as acc += (p * sy[g, j]) * sx[g, i], the group's
// scales of the lane's four columns j and its row i.
template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void k_grouped_kernel(KGroupedArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    const WsLayout L = ws_layout(p.G, 0);
    const int64_t* offs = (const int64_t*)(p.ws + L.offsets);
    const int32_t* order = (const int32_t*)(p.ws + L.order);
    const int n_it = p.Mw / C::BM, n_jt = p.Nw / C::BN;
    const int per_e = n_it * n_jt;
    const int item = block_to_item(blockIdx.x);
    if (item >= p.G * per_e) return;
    const int rank = item / per_e;
    int it, jt;
    item_to_tiles(item - rank * per_e, n_it, n_jt, it, jt);
    const int e = order[rank];
    const int64_t t0 = offs[e];
    const int64_t te = max((int64_t)0, min(offs[e + 1], offs[p.G]) - t0);
    const int i0 = it * C::BM, j0 = jt * C::BN;
    const uint32_t x_row = (uint32_t)p.Mw * C::ESZ, y_row = (uint32_t)p.Nw * C::ESZ;
    auto rx = make_rsrc((const char*)p.X + t0 * x_row, (uint32_t)(te * x_row));
    auto ry = make_rsrc((const char*)p.dY + t0 * y_row, (uint32_t)(te * y_row));
    const int nks = (int)((te + C::KSTEP - 1) / C::KSTEP);

    v4f acc[C::NB][C::MB];
#pragma unroll
    for (int i = 0; i < C::NB; ++i)
#pragma unroll
        for (int j = 0; j < C::MB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int r16 = lane & 15, g4 = (lane >> 4) * 4;
    // fp8: the scale DMA of this wave, fixed per tile.  Waves below BM / 64 load
    // the X scales of the tile's BM columns, the others the dY scales; scale row
    // (group) groups[e] + ks, one 4-byte DMA per thread per stage.  A group past
    // the scale arrays reads 0 (MOEGG_FLAG_SCALE_GROUPS).
    __amdgpu_buffer_rsrc_t rss = make_rsrc(nullptr, 0);
    uint32_t ss_voff = 0, ss_step = 0, ss_dst = 0;
    if constexpr (C::E8M0) {
        // even waves: the tile's 256 X scale bytes of the group (4 per lane), odd
        // waves: its 256 dY scale bytes; the waves of a parity write the same
        // bytes to the same slots
        const int64_t g0 = ((const int64_t*)(p.ws + L.groups))[e];
        const bool xs = (wave & 1) == 0;
        const uint32_t srow = xs ? (uint32_t)p.Mw : (uint32_t)p.Nw;
        rss = xs ? make_rsrc(p.X_scale, (uint32_t)(p.scale_groups * srow))
                 : make_rsrc(p.dY_scale, (uint32_t)(p.scale_groups * srow));
        const int col = (xs ? i0 : j0) + lane * 4;
        ss_voff = g0 < p.scale_groups ? (uint32_t)(g0 * srow) + col : 0x80000000u;
        ss_step = srow;
        ss_dst = C::A_BYTES + C::B_BYTES + (xs ? 0 : C::BM);
    } else if constexpr (C::FP8) {
        const int64_t g0 = ((const int64_t*)(p.ws + L.groups))[e];
        const bool xs = wave < C::BM / 64;
        const uint32_t srow = xs ? (uint32_t)p.Mw * 4 : (uint32_t)p.Nw * 4;
        rss = xs ? make_rsrc(p.X_scale, (uint32_t)(p.scale_groups * srow))
                 : make_rsrc(p.dY_scale, (uint32_t)(p.scale_groups * srow));
        const int col = (xs ? i0 : j0) + (xs ? wave : wave - C::BM / 64) * 64 + lane;
        // a group index past the arrays is parked past the buffer and reads 0
        ss_voff = g0 < p.scale_groups ? (uint32_t)(g0 * srow) + col * 4 : 0x80000000u;
        ss_step = srow;
        ss_dst = C::A_BYTES + C::B_BYTES + wave * 256;
    }
    auto issue = [&](int ks, char* __restrict__ base) {
        load_tile_mn<C, C::BM * C::ESZ>(rx, x_row, ks * C::KSTEP, i0 * C::ESZ, base, C::A_LOADS);
        load_tile_mn<C, C::BN * C::ESZ>(ry, y_row, ks * C::KSTEP, j0 * C::ESZ, base + C::A_BYTES, C::B_LOADS);
        if constexpr (C::FP8) {
            const uint32_t v = ss_voff >= 0x80000000u ? ss_voff : ss_voff + (uint32_t)ks * ss_step;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rss, (MOEGG_LDS void*)(base + ss_dst), 4, v, 0, 0, 0);
        }
    };
    // Same pipeline as the contiguous kernel: loads run STAGES - 1 steps ahead,
    // the DMAs of a step are issued after the first MFMA block of the step
    // STAGES - 1 earlier, one vmcnt wait and one barrier per step.  An expert
    // with no rows runs no steps and writes zeros.
    if (nks > 0) {
        constexpr int S = C::STAGES;
#pragma unroll
        for (int s = 0; s < S - 1; ++s) issue(min(s, nks - 1), lds + s * C::STAGE_BYTES);
        wait_vmcnt<(S - 2) * C::OPS>();
        __syncthreads();
        int cur = 0, free = S - 1;
        // the read stage and the DMA stage of a step differ (see TileGemm::step)
        auto step = [&](const char* __restrict__ tx, char* __restrict__ wr, int next) {
            const char* ty = tx + C::A_BYTES;
            if constexpr (C::E8M0) {
                // the group's scale bytes go to the MFMA: scale_a (dY, the A operand)
                // is each lane's dY column byte, scale_b (X) its X column byte, and the
                // MFMA adds the scaled group straight into acc: no VALU work per group.
                // (Adding a zero-started group partial to acc on the VALU instead gives
                // the fp32-scale kernel's bits but costs 11 %.)
                const MOEGG_LDS unsigned char* sxb = (const MOEGG_LDS unsigned char*)(ty + C::B_BYTES);
                const MOEGG_LDS unsigned char* syb = sxb + C::BM;
                v8i xa[C::MB];
                int sxj[C::MB];
#pragma unroll
                for (int j = 0; j < C::MB; ++j) {
                    xa[j] = frag_mn_fp8<C::BM>(tx, wm * C::WTM + j * 16);
                    sxj[j] = sxb[wm * C::WTM + j * 16 + r16];
                }
                auto fragy = [&](int i) { return frag_mn_fp8<C::BN>(ty, wn * C::WTN + i * 16); };
                v8i yb[2];
                yb[0] = fragy(0);
                static_for<0, C::NB>([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    if constexpr (i + 1 < C::NB) yb[(i + 1) & 1] = fragy(i + 1);
                    const int syi = syb[wn * C::WTN + i * 16 + r16];
#pragma unroll
                    for (int j = 0; j < C::MB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(yb[i & 1], xa[j], acc[i][j], 0,
                                                                                     0, 0, syi, 0, sxj[j]);
                    if constexpr (i == 0) issue(next, wr);
                    __builtin_amdgcn_sched_barrier(0);
                });
            } else if constexpr (C::FP8) {
                // this wave's X fragments and row scales, then the dY blocks one ahead
                // of their MFMAs; each block's partials promoted with the group's scales
                const float* sx = (const float*)(ty + C::B_BYTES);
                const float* sy = sx + C::BM;
                v8i xa[C::MB];
                float sxj[C::MB];
#pragma unroll
                for (int j = 0; j < C::MB; ++j) {
                    xa[j] = frag_mn_fp8<C::BM>(tx, wm * C::WTM + j * 16);
                    sxj[j] = sx[wm * C::WTM + j * 16 + r16];
                }
                auto fragy = [&](int i) { return frag_mn_fp8<C::BN>(ty, wn * C::WTN + i * 16); };
                v8i yb[2];
                yb[0] = fragy(0);
                v4f pp[C::MB];
                static_for<0, C::NB>([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    if constexpr (i + 1 < C::NB) yb[(i + 1) & 1] = fragy(i + 1);
                    const v4f syi = *(const MOEGG_LDS v4f*)(sy + wn * C::WTN + i * 16 + g4);
#pragma unroll
                    for (int j = 0; j < C::MB; ++j) pp[j] = mfma_fp8(yb[i & 1], xa[j], v4f{0.f, 0.f, 0.f, 0.f});
                    if constexpr (i == 0) issue(next, wr);
#pragma unroll
                    for (int j = 0; j < C::MB; ++j) {
                        const v4f q = pp[j] * syi;
                        acc[i][j].x = __builtin_fmaf(q.x, sxj[j], acc[i][j].x);
                        acc[i][j].y = __builtin_fmaf(q.y, sxj[j], acc[i][j].y);
                        acc[i][j].z = __builtin_fmaf(q.z, sxj[j], acc[i][j].z);
                        acc[i][j].w = __builtin_fmaf(q.w, sxj[j], acc[i][j].w);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            } else {
                // both K halves of this wave's X fragments, then the dY blocks one
                // ahead of their MFMAs
                v4i xa[2][C::MB];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int j = 0; j < C::MB; ++j) xa[kk][j] = frag_mn_bf16<C::BM * 2>(tx, wm * C::WTM + j * 16, kk);
                auto fragy = [&](int i, int kk) { return frag_mn_bf16<C::BN * 2>(ty, wn * C::WTN + i * 16, kk); };
                v4i yb[2];
                yb[0] = fragy(0, 0);
                static_for<0, 2 * C::NB>([&](auto U) {
                    constexpr int u = decltype(U)::value, i = u >> 1, kk = u & 1;
                    if constexpr (u + 1 < 2 * C::NB) yb[(u + 1) & 1] = fragy((u + 1) >> 1, (u + 1) & 1);
#pragma unroll
                    for (int j = 0; j < C::MB; ++j) acc[i][j] = mfma_bf16(yb[u & 1], xa[kk][j], acc[i][j]);
                    if constexpr (u == 0) issue(next, wr);
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
        };
        for (int ks = 0; ks < nks; ++ks) {
            __builtin_amdgcn_s_setprio(1);
            step(lds + cur * C::STAGE_BYTES, lds + free * C::STAGE_BYTES, min(ks + S - 1, nks - 1));
            __builtin_amdgcn_s_setprio(0);
            wait_vmcnt<(S - 2) * C::OPS>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            compiler_fence();
            free = cur;
            cur = cur + 1 == S ? 0 : cur + 1;
        }
        wait_vmcnt<0>();
    }
    // fp32 epilogue (lane holds dW[i][j..j+3]) through LDS in two passes of
    // BM / 2 rows, which is what the ring holds: the waves owning those rows
    // write them as [BM/2][BN] fp32 with 16-byte chunks XOR-swizzled by
    // row & 15, then every lane stores 16 bytes of a whole row, so each store
    // instruction writes 1 KB of consecutive bytes instead of 64-byte pieces of
    // 16 rows.  The first barrier also covers every wave's last DMAs.
    static_assert(C::WAVES_M % 2 == 0 && (C::BM / 2) * C::BN * 4 <= C::LDS_BYTES, "epilogue passes");
    constexpr int RB = C::BN * 4, CPR = RB / 16, HALF_ROWS = C::BM / 2;
    static_assert(CPR >= 16 && C::THREADS % CPR == 0, "row swizzle");
    const int g = lane >> 4;
    float* out = p.dW + (size_t)e * p.Mw * p.Nw;
    const int c = tid % CPR;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __syncthreads();
        if (wm / (C::WAVES_M / 2) == h) {
#pragma unroll
            for (int j = 0; j < C::MB; ++j) {
                const int row = (wm % (C::WAVES_M / 2)) * C::WTM + j * 16 + r16;
#pragma unroll
                for (int n = 0; n < C::NB; ++n) {
                    const int chunk = ((wn * C::WTN + n * 16 + 4 * g) >> 2) ^ (row & 15);
                    *(MOEGG_LDS v4f*)(lds + row * RB + chunk * 16) = acc[n][j];
                }
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int r0 = 0; r0 < HALF_ROWS; r0 += C::THREADS / CPR) {
            const int row = r0 + tid / CPR;
            const v4f v = *(const MOEGG_LDS v4f*)(lds + row * RB + ((c ^ (row & 15)) << 4));
            *(v4f*)(out + (size_t)(i0 + h * HALF_ROWS + row) * p.Nw + j0 + c * 4) = v;
        }
    }
}

// ---------------------------------------------------------------- configs

using KGroupedCfg = KCfg<256, 256, 4, 2, 2>;
using KGroupedFp8Cfg = KCfg<256, 256, 4, 2, 2, true>;
using KGroupedE8Cfg = KCfg<256, 256, 4, 2, 2, true, true>;

// Raise a kernel's dynamic LDS limit once per process (it is a function
// attribute, not a stream operation).
template <auto Kernel>
static hipError_t allow_lds(int bytes) {
    static hipError_t once =
        hipFuncSetAttribute((const void*)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return once;
}

template <class C, bool B_KN, int SWIGLU = 0>
static hipError_t launch_one(const ContigArgs& a, int grid, hipStream_t s) {
    auto k = grouped_gemm_kernel<C, B_KN, SWIGLU>;
    hipError_t err = allow_lds<grouped_gemm_kernel<C, B_KN, SWIGLU>>(C::LDS_BYTES);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

static int round256(int64_t x) { return (int)((x + 255) / 256 * 256); }

// Launch the contiguous GEMM for tile height block_m.  0 (the height the
// device chose) and per-expert heights run in one launch of the auto kernel;
// an explicit 64, 128 or 256 runs that height's own kernel, which writes
// nothing unless the schedule used the same height.
template <bool FP8, bool B_KN, bool E8, bool W4 = false, int SW = 0>
static hipError_t launch_contig_t(const ContigArgs& a, int64_t rows_total, int block_m, hipStream_t s) {
    const int64_t n_ct = a.N / 256;
    auto grid_for = [&](int q) { return round256(((rows_total + q - 1) / q + a.G) * n_ct); };
    if (block_m == MOEGG_BLOCK_M_PER_EXPERT || block_m == 0) {
        ContigArgs b = a;
        b.req_block_m = block_m;
        constexpr int lds = std::max({Contig256<FP8, E8, W4>::LDS_BYTES, Contig128<FP8, E8, W4>::LDS_BYTES,
                                      Contig64<FP8, E8, W4>::LDS_BYTES});
        hipError_t err = allow_lds<grouped_gemm_auto_kernel<FP8, B_KN, E8, W4, SW>>(lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((grouped_gemm_auto_kernel<FP8, B_KN, E8, W4, SW>), dim3(grid_for(64)), dim3(512), lds,
                           s, b);
        return hipGetLastError();
    }
    if (block_m == 256) return launch_one<Contig256<FP8, E8, W4>, B_KN, SW>(a, grid_for(256), s);
    if (block_m == 128) return launch_one<Contig128<FP8, E8, W4>, B_KN, SW>(a, grid_for(128), s);
    return launch_one<Contig64<FP8, E8, W4>, B_KN, SW>(a, grid_for(64), s);
}

hipError_t launch_contiguous(const ContigArgs& a, bool fp8, bool e8m0, bool w4, bool b_kn, int64_t rows_total,
                             int block_m, hipStream_t s) {
    if (w4) return b_kn ? hipErrorInvalidValue : launch_contig_t<true, false, true, true>(a, rows_total, block_m, s);
    if (fp8 && e8m0) return b_kn ? launch_contig_t<true, true, true>(a, rows_total, block_m, s)
                                 : launch_contig_t<true, false, true>(a, rows_total, block_m, s);
    if (fp8) return b_kn ? launch_contig_t<true, true, false>(a, rows_total, block_m, s)
                         : launch_contig_t<true, false, false>(a, rows_total, block_m, s);
    return b_kn ? launch_contig_t<false, true, false>(a, rows_total, block_m, s)
                : launch_contig_t<false, false, false>(a, rows_total, block_m, s);
}

hipError_t launch_contiguous_swiglu(const ContigArgs& a, bool fp8, bool w4, int64_t rows_total, int block_m,
                                    hipStream_t s) {
    const bool q = a.C_scale != nullptr;      // e4m3 H with fp32 scales
    if (w4) return q ? launch_contig_t<true, false, true, true, 2>(a, rows_total, block_m, s)
                     : launch_contig_t<true, false, true, true, 1>(a, rows_total, block_m, s);
    if (fp8) return q ? launch_contig_t<true, false, false, false, 2>(a, rows_total, block_m, s)
                      : launch_contig_t<true, false, false, false, 1>(a, rows_total, block_m, s);
    return q ? launch_contig_t<false, false, false, false, 2>(a, rows_total, block_m, s)
             : launch_contig_t<false, false, false, false, 1>(a, rows_total, block_m, s);
}

int masked_block_m() { return Masked128<false>::BM; }
int masked_block_n() { return Masked128<false>::BN; }

template <bool FP8, bool B_KN, bool E8 = false, bool W4 = false>
static hipError_t launch_masked_t(const ContigArgs& a, hipStream_t s) {
    constexpr int lds = std::max(Masked128<FP8, E8, W4>::LDS_BYTES, Masked64<FP8, E8, W4>::LDS_BYTES);
    static_assert(2 * lds <= 160 * 1024, "two workgroups per CU");
    hipError_t err = allow_lds<grouped_gemm_masked_kernel<FP8, B_KN, E8, W4>>(lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((grouped_gemm_masked_kernel<FP8, B_KN, E8, W4>), dim3(a.G * (a.N / 128)), dim3(512), lds, s,
                       a);
    return hipGetLastError();
}

hipError_t launch_masked(const ContigArgs& a, bool fp8, bool e8m0, bool w4, bool b_kn, hipStream_t s) {
    if (w4) return b_kn ? hipErrorInvalidValue : launch_masked_t<true, false, true, true>(a, s);
    if (e8m0) return b_kn ? launch_masked_t<true, true, true>(a, s) : launch_masked_t<true, false, true>(a, s);
    if (fp8) return b_kn ? launch_masked_t<true, true>(a, s) : launch_masked_t<true, false>(a, s);
    return b_kn ? launch_masked_t<false, true>(a, s) : launch_masked_t<false, false>(a, s);
}

template <class C>
static hipError_t launch_k_grouped_t(const KGroupedArgs& a, hipStream_t s) {
    auto k = k_grouped_kernel<C>;
    hipError_t err = allow_lds<k_grouped_kernel<C>>(C::LDS_BYTES);
    if (err != hipSuccess) return err;
    const int64_t items = (int64_t)a.G * (a.Mw / C::BM) * (a.Nw / C::BN);
    hipLaunchKernelGGL(k, dim3(round256(items)), dim3(C::THREADS), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

hipError_t launch_mlp_fused(const MlpArgs& a, int n_workgroups, hipStream_t s) {
    using C = Contig256<true>;
    hipError_t err = allow_lds<expert_mlp_fused_kernel>(C::LDS_BYTES);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(expert_mlp_fused_kernel, dim3(n_workgroups), dim3(C::THREADS), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

hipError_t launch_k_grouped(const KGroupedArgs& a, bool fp8, bool e8m0, hipStream_t s) {
    if (e8m0) return launch_k_grouped_t<KGroupedE8Cfg>(a, s);
    return fp8 ? launch_k_grouped_t<KGroupedFp8Cfg>(a, s) : launch_k_grouped_t<KGroupedCfg>(a, s);
}

}  // namespace moegg
