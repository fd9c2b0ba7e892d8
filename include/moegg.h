/*
 * moegg.h -- C ABI of the MI355X (gfx950) MoE grouped GEMM library, libmoegg.so.
 *
 * The operation: expert e multiplies its m_e routed rows [m_e, K] by its own
 * weight B_e [K, N].  N and K are shared by all experts.  The counts m_e are
 * ragged, skewed and often zero.  Gathering each expert's tokens into one GEMM
 * alters how the work is tiled; every output is still the same product.  Only
 * M is grouped, because experts share one N and one K.  (DeepGEMM
 * grouped/masked MoE GEMM record, "Arithmetic intensity".)
 *
 * Conventions for every call below:
 *   - Pointers are device pointers unless the name starts with h_.
 *   - `stream` is a hipStream_t (NULL = the default stream).
 *   - Compute calls are asynchronous on `stream`.  They never allocate, never
 *     synchronize, and never copy to the host, so they can be captured in a
 *     HIP graph.  Only the *_read calls synchronize.
 *   - The caller owns every buffer, including the workspace.  The library
 *     keeps no pointer after a call returns.
 *   - Argument errors are found on the host before anything is enqueued.  The
 *     call then returns an error code and launches nothing.
 *   - Bad counts on the device cannot be reported without a host round trip.
 *     The device clamps them, never reads or writes out of bounds, and sets a
 *     bit in moegg_stats_t.error_flags.
 *   - One workspace per stream in flight.  Calls that share a workspace must
 *     be ordered.
 */
#ifndef MOEGG_H
#define MOEGG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOEGG_OK = 0,
    MOEGG_ERR_INVALID_ARG = 1,   /* null pointer, bad size or count           */
    MOEGG_ERR_UNSUPPORTED = 2,   /* shape or option the library does not cover */
    MOEGG_ERR_WORKSPACE = 3,     /* workspace missing or too small            */
    MOEGG_ERR_HIP = 4            /* a HIP runtime call failed                 */
} moegg_status_t;

/* Operand storage type.  MOEGG_FP8_E4M3 is OCP e4m3fn (max 448, no inf) with
 * fp32 block scales, promoted into the fp32 accumulator group by group.
 * MOEGG_FP8_E4M3_E8M0 is the same operands with power-of-two block scales
 * stored as E8M0 exponent bytes (value 2^(b - 127); 255 is NaN), the packed
 * UE8M0 scale format the DeepGEMM record names for SM100.  On gfx950 the MFMA
 * applies them itself (V_MFMA_SCALE_F32_16X16X128_F8F6F4), so nothing is
 * promoted on the VALU.  Its activation scales are stored transposed:
 * [K/128, rows] (DeepGEMM's MN-major scale layout), four rows per 32-bit word.
 * Contiguous and masked layouts.
 * MOEGG_FP8_E4M3_FP4_E2M1 is the low-precision-weight case the DeepGEMM
 * record lists for SM100 (FP8 x FP4): activations as for
 * MOEGG_FP8_E4M3_E8M0, weights as OCP E2M1 (fp4: sign, 2 exponent bits with
 * bias 1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6) packed two per
 * byte, element 2i in the low nibble, stored [G, N, K/2] (MOEGG_B_NK) or in
 * its panels [G, N/P, K/128, P, 64] (MOEGG_B_NK_PANEL), with E8M0
 * weight-block scales [G, K/128, N/128].  The same gfx950 MFMA takes the fp4
 * operand directly.  Contiguous and masked layouts and the SwiGLU call. */
/* MOEGG_FP8_E4M3_SCALE_KM is MOEGG_FP8_E4M3 with the fp32 activation
 * scales stored transposed, [K/128, rows] (the record's note that SM100 wants
 * a transposed LHS scale layout; here for fp32 scales).  One K step's scales
 * of a tile's rows are then contiguous: the kernel fetches them as a few
 * cache lines instead of one line per row.  Same arithmetic as
 * MOEGG_FP8_E4M3.  Contiguous and masked layouts and the SwiGLU call. */
typedef enum {
    MOEGG_BF16 = 0,
    MOEGG_FP8_E4M3 = 1,
    MOEGG_FP8_E4M3_E8M0 = 2,
    MOEGG_FP8_E4M3_FP4_E2M1 = 3,
    MOEGG_FP8_E4M3_SCALE_KM = 4
} moegg_dtype_t;

/* How each expert's weight B_e is stored.
 *   MOEGG_B_KN: B[G, K, N], N contiguous.
 *   MOEGG_B_NK: B[G, N, K], K contiguous.
 *   MOEGG_B_KN_PANEL: B[G, N/P, K, P]: the columns in panels of P, each panel
 *     K rows of P contiguous elements, panels back to back.
 *   MOEGG_B_NK_PANEL: B[G, N/P, K/S, P, S], S = one K step: 128 bytes of K
 *     (64 bf16, 128 e4m3), or 64 bytes (128 packed fp4 codes): each panel of
 *     P columns stored one K step at a time, so the weights one tile loads
 *     per K step are one contiguous block of whole cache lines.
 * P is the column tile of the call: 256 for the contiguous and SwiGLU calls,
 * 128 for the masked call.  The panel layouts are one-time weight repacks,
 * like the choice between [G,K,N] and [G,N,K]; they change where a weight
 * sits, not the arithmetic.  The fp8 block scales are [G, K/128, N/128] in
 * every layout. */
typedef enum {
    MOEGG_B_KN = 0,
    MOEGG_B_NK = 1,
    MOEGG_B_KN_PANEL = 2,
    MOEGG_B_NK_PANEL = 3
} moegg_b_layout_t;

/* error_flags bits */
#define MOEGG_FLAG_NEGATIVE_COUNT  0x1u  /* a count < 0 was read as 0                 */
#define MOEGG_FLAG_ROWS_OVERFLOW   0x2u  /* segments ran past rows_total / T; truncated */
#define MOEGG_FLAG_COUNT_OVER_CAP  0x4u  /* a masked count > cap was read as cap      */
#define MOEGG_FLAG_BAD_EXEMPLAR    0x8u  /* an exemplar named an invalid block_m      */
#define MOEGG_FLAG_SCALE_GROUPS    0x10u /* K-grouped fp8: the histogram needs more scale
                                            groups than the scale arrays hold; the
                                            missing groups' scales read as 0           */
#define MOEGG_FLAG_SYNC_TIMEOUT    0x20u /* fused expert MLP: a down-projection tile gave up
                                            waiting for its H rows (bounded wait); its
                                            output rows are unspecified               */

/* block_m value for per-expert tile heights: every expert gets 256-row tiles,
 * and its remainder rows one tile of the smallest height in {64, 128, 256}
 * that holds them.  The padding page's "Adapt kernels without adding a CPU
 * stall" section asks for per-histogram kernel choice on the device; this
 * choice is per expert.  The tile list is the 256-row list, ordered: tiles
 * with more than 128 valid rows, then tiles with 65..128, then 1..64, each
 * group in expert order. */
#define MOEGG_BLOCK_M_PER_EXPERT (-1)

/* Tile heights the schedule accounts for, in P_at[] order. */
#define MOEGG_NUM_Q 6                    /* q = 8, 16, 32, 64, 128, 256 */

/*
 * Padding accounting, written on the device by every scheduled call.  It
 * follows "MoE GroupGEMM padding under expert skew":
 *   - section "Calculate padded token columns": U, P(q), P - U;
 *   - section "Summarize skew without losing the histogram": effective
 *     experts = U^2 / sum_sq, derived on the host from the exact integers;
 *   - section "Grouped execution does not require padded experts": capacity
 *     padding and tail padding are kept apart.
 */
typedef struct {
    int64_t U;               /* useful rows: sum of the (clamped) counts                     */
    int64_t P_exec;          /* rows the MFMAs executed: each tile's valid rows rounded up to */
                             /* the kernel's 16-row MFMA block (= tail padding + U)           */
    int64_t tiles;           /* entries in the tile list (M tiles of height block_m)          */
    int64_t active;          /* experts with a nonzero count                                  */
    int64_t sum_sq;          /* sum of squared counts                                         */
    int64_t capacity_rows;   /* layout rows holding no valid row (alignment gaps, unused cap) */
    int64_t P_at[MOEGG_NUM_Q]; /* P(q) = sum over active experts of q * ceil(m_e / q)         */
    int32_t block_m;         /* tile height used                                              */
    uint32_t error_flags;    /* MOEGG_FLAG_* bits                                             */
} moegg_stats_t;

/*
 * Ratios derived from one moegg_stats_t, for reports ("MoE GroupGEMM padding
 * under expert skew": section "Calculate padded token columns" for the padding
 * fraction (P - U) / P and the useful share U / P; section "Summarize skew
 * without losing the histogram" for effective experts U^2 / sum m_e^2; section
 * "Padding is not the whole cost model" for physical versus effective work).
 * Each is computed from the exact integers in extended precision and rounded
 * once to double.  A ratio whose denominator is 0 reads 0.
 */
typedef struct {
    double effective_experts;             /* U^2 / sum_sq                             */
    double padding_fraction[MOEGG_NUM_Q]; /* (P(q) - U) / P(q), q = 8 .. 256          */
    double useful_share[MOEGG_NUM_Q];     /* U / P(q): the aggregate M-occupancy      */
    double exec_padding_fraction;         /* (P_exec - U) / P_exec: rows the MFMAs ran */
                                          /* without a valid row                       */
    double physical_over_effective;       /* P_exec / U: physical / effective work     */
} moegg_report_t;

/* Fill *h_out from *h_stats.  Pure host function (no stream, no device).
 * MOEGG_ERR_INVALID_ARG for NULL pointers or negative counts in *h_stats. */
moegg_status_t moegg_stats_report(const moegg_stats_t* h_stats, moegg_report_t* h_out);

/* One entry of the device tile list: expert, tile index within the expert,
 * first row of the tile in A/C, and valid rows (1..block_m). */
typedef struct { int32_t expert, tile, row_start, rows_valid; } moegg_tile_t;

/* Library version, (major << 16) | minor. */
int moegg_version(void);

/* Short text for a status code (static storage). */
const char* moegg_status_string(moegg_status_t status);

/*
 * Workspace bytes for a problem with G experts (G = 1..4096) and up to
 * max_rows rows of A (rows_total for the contiguous layout, G * cap for the
 * masked one, T for the K-grouped one).  Pure host function.  Returns 0 for
 * invalid arguments.
 */
size_t moegg_workspace_bytes(int G, int64_t max_rows);

/*
 * Device-side scheduler alone: counts -> tile list + stats in `ws`, with no
 * host round trip.
 *
 * For every expert e with m_e > 0 and every i < ceil(m_e / block_m) it emits
 *     {e, i, seg_off[e] + i * block_m, min(block_m, m_e - i * block_m)}
 * in expert-ascending, tile-ascending order, where
 *     seg_off[e] = sum_{j<e} align_up(m_j, seg_align).
 * Empty experts emit nothing, so their weights are never loaded.  This is
 * the variable-M work list of "Grouped execution does not require padded
 * experts", built from the actual counts.
 *
 * block_m must be 64, 128 or 256, 0 to let the device choose one height
 * (see moegg_grouped_gemm_contiguous), or MOEGG_BLOCK_M_PER_EXPERT.  N is the output width of the GEMM the
 * schedule will feed: the choice rule counts its 256-wide column tiles.
 * seg_align >= 1.  Segments are truncated at rows_total (flag
 * MOEGG_FLAG_ROWS_OVERFLOW).
 */
moegg_status_t moegg_schedule(const int32_t* m_sizes, int G, int64_t rows_total, int seg_align,
                              int block_m, int N, void* ws, size_t ws_bytes, void* stream);

/*
 * Distribution-aware tile-height selection ("MoE GroupGEMM padding under
 * expert skew", section "Adapt kernels without adding a CPU stall": sort and
 * normalize the per-expert counts, match them against exemplars tuned
 * offline, and keep neighbouring histograms from flipping the kernel).
 *
 * An exemplar describes one histogram by
 *   size_class  4 * floor(log2 U) + the two bits of U below its leading one
 *               (quarter-octave steps of the row count U; 0 when U = 0);
 *   lorenz[i]   floor(65536 * S(k_i) / U), i = 0..7, where S(k) is the sum of
 *               the k largest counts and k_i = ceil(G * (i + 1) / 8): the share
 *               of the rows held by the top eighth, quarter, ... of experts
 *               (all 0 when U = 0);
 * and names the configuration measured fastest for it (block_m: 64, 128,
 * 256 or MOEGG_BLOCK_M_PER_EXPERT).
 */
typedef struct {
    int32_t size_class;
    int32_t lorenz[8];
    int32_t block_m;
} moegg_exemplar_t;

#define MOEGG_MAX_EXEMPLARS 256
#define MOEGG_EXEMPLAR_SIZE_WEIGHT 8192   /* distance per quarter-octave of U */

/*
 * moegg_schedule with the tile height chosen by exemplar matching on the
 * device.  The histogram's descriptor (as above, from the clamped counts)
 * is compared with each exemplar by
 *     D = sum_i |lorenz[i] - ex.lorenz[i]|
 *         + MOEGG_EXEMPLAR_SIZE_WEIGHT * |size_class - ex.size_class|,
 * and the nearest exemplar wins (ties: lowest index).  Hysteresis: `ws`
 * remembers the exemplar the previous call on it chose; that one is kept
 * while its distance is at most the nearest one's plus `hysteresis`.  A
 * workspace that no call of this kind has used carries no choice (a 64-bit
 * tag marks a valid one).  The chosen exemplar's block_m then drives the tile
 * list exactly as in moegg_schedule; stats block_m reports it.  If it is not
 * a valid block_m, the cost rule of moegg_grouped_gemm_contiguous decides
 * (for output width N) and error_flags gets MOEGG_FLAG_BAD_EXEMPLAR.
 * Arguments other than the three below are those of moegg_schedule.
 *   exemplars  device array of n_exemplars entries (1..MOEGG_MAX_EXEMPLARS),
 *              read during the call; caller-owned.
 *   hysteresis >= 0, in distance units.
 * Graph-capturable: nothing leaves the device.  Calls that share a
 * workspace must be ordered (the remembered choice is part of it).
 */
moegg_status_t moegg_schedule_exemplar(const int32_t* m_sizes, int G, int64_t rows_total, int seg_align, int N,
                                       const moegg_exemplar_t* exemplars, int n_exemplars, int hysteresis,
                                       void* ws, size_t ws_bytes, void* stream);

/* What the last moegg_schedule_exemplar call on a workspace saw and chose. */
typedef struct {
    int32_t exemplar;        /* index of the chosen exemplar                    */
    int32_t size_class;      /* the histogram's descriptor, as defined above    */
    int32_t lorenz[8];
    int64_t distance;        /* distance from the histogram to the chosen exemplar */
} moegg_selection_t;

/* Copy the selection of the last moegg_schedule_exemplar call on `ws` to
 * the host.  Synchronizes `stream`.  MOEGG_ERR_INVALID_ARG if no such call
 * has used `ws`. */
moegg_status_t moegg_selection_read(const void* ws, moegg_selection_t* h_out, void* stream);

/*
 * M-grouped contiguous layout (DeepGEMM record, "Workarounds": prefill and
 * training, where token counts are known).
 *   A        [rows_total, K], row-major.  Expert e's rows start at seg_off[e],
 *            as in moegg_schedule.  seg_align = 1 packs them back to back.  A
 *            larger seg_align puts every segment start at a multiple of it.
 *   A_scale  MOEGG_FP8_E4M3: fp32 [rows_total, K/128], one scale per 1x128
 *            group.  MOEGG_FP8_E4M3_SCALE_KM: the same scales as fp32
 *            [K/128, rows_total].  MOEGG_FP8_E4M3_E8M0: E8M0 bytes
 *            [K/128, rows_total] (transposed).  NULL for bf16.
 *   B        [G, K, N] or [G, N, K] (b_layout), same dtype as A.
 *            MOEGG_FP8_E4M3_FP4_E2M1: packed E2M1 bytes [G, N, K/2].
 *   B_scale  MOEGG_FP8_E4M3 and MOEGG_FP8_E4M3_SCALE_KM: fp32
 *            [G, K/128, N/128], one per 128x128 block.
 *            MOEGG_FP8_E4M3_E8M0 and MOEGG_FP8_E4M3_FP4_E2M1: E8M0 bytes,
 *            same shape.  NULL for bf16.
 *   C        bf16 [rows_total, N], row-major.  Only the rows of valid
 *            segments are written.  Other rows keep their contents.
 *   m_sizes  int32 [G] on the device.
 * Computes, for each valid row R of expert e:
 *     C[R, n] = bf16_rne( sum_k A[R, k] * B_e[k, n] )
 * with fp32 accumulation.  For fp8, each 128-wide K group's fp32 partial sum
 * is multiplied by A_scale[R, k/128] * B_scale[e, k/128, n/128] and added to
 * the fp32 accumulator.  With E8M0 scales the MFMA scales its operands by
 * the two powers of two instead: the same value up to fp32 rounding order.
 * Constraints: K % 128 == 0 and N % 256 == 0 for fp8.  K % 64 == 0 and
 * N % 256 == 0 for bf16.  E8M0 scales also need N % 512 == 0, N <= 32768
 * and rows_total % 4 == 0 (UNSUPPORTED otherwise); scales stored [K/128,
 * rows_total] (E8M0, MOEGG_FP8_E4M3_SCALE_KM) must span at most 4 GiB
 * (UNSUPPORTED otherwise); fp4 weights also need
 * b_layout = MOEGG_B_NK (UNSUPPORTED otherwise).  16-byte aligned
 * operands, 4-byte aligned scales.  G = 1..4096.
 * block_m: 64, 128 or 256; 0 = choose one height on the device from the
 * histogram; MOEGG_BLOCK_M_PER_EXPERT = per-expert heights (see its
 * definition), stats block_m then reads MOEGG_BLOCK_M_PER_EXPERT.
 * Every height skips whole 16-row MFMA blocks past a tile's valid rows, so
 * the executed rows are P(16) for all of them.  What differs is how many
 * 256x(block_m) tiles there are and how full the last round of tiles is on
 * 256 CUs.  The device choice minimizes
 *     cost(q) = ceil(tiles(q) * (N / 256) / 256) * (q + 64)
 * over q in {64, 128, 256}, with ties going to the larger q (better weight
 * reuse), and compares it with per-expert heights, costed class by class:
 *     cost_pe = sum over c of ceil(n_c * (N / 256) / 256) * (q_c + 64)
 * where n_c counts the 256-row tiles (q_c = 256), the remainders of 65..128
 * rows (q_c = 128) and of 1..64 rows (q_c = 64).  Per-expert heights are
 * chosen only when strictly cheaper; stats block_m then reads
 * MOEGG_BLOCK_M_PER_EXPERT.  Padding alone does not pick the kernel
 * ("Padding is not the whole cost model", MoE GroupGEMM padding page).  The
 * GEMM is one launch whose grid size comes from host arguments alone (sized
 * for the longest tile list, 64-row tiles; workgroups past the list the
 * device chose exit at once), so the call is graph-capturable.
 */
moegg_status_t moegg_grouped_gemm_contiguous(
    const void* A, const void* A_scale, const void* B, const void* B_scale, void* C,
    const int32_t* m_sizes, int G, int64_t rows_total, int K, int N, int seg_align,
    moegg_dtype_t dtype, moegg_b_layout_t b_layout, int block_m,
    void* ws, size_t ws_bytes, void* stream);

/*
 * moegg_grouped_gemm_contiguous for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture that may not call
 * hipMalloc, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, computation, constraints and errors as
 * moegg_grouped_gemm_contiguous, without ws and ws_bytes.  The scheduler's
 * workspace is a fixed array of MOEGG_NOALLOC_SCRATCH_BYTES in each GPU's
 * memory, held by the library until the process ends; problems whose
 * workspace (moegg_workspace_bytes(G, rows_total)) exceeds it return
 * MOEGG_ERR_WORKSPACE before anything is enqueued.  The call allocates
 * nothing: on its first use on a GPU it looks up the array's address there
 * (the calling thread's current device, which `stream` must belong to).
 * Every call on one GPU uses the same array and each call rewrites what the
 * GEMM reads, so calls in order on one GPU are independent; calls that overlap
 * on one GPU (concurrent streams, several threads) race.  The stats and tile
 * list it leaves there are not readable through moegg_stats_read.
 */
#define MOEGG_NOALLOC_SCRATCH_BYTES (1u << 20)

moegg_status_t moegg_grouped_gemm_contiguous_noalloc(
    const void* A, const void* A_scale, const void* B, const void* B_scale, void* C,
    const int32_t* m_sizes, int G, int64_t rows_total, int K, int N, int seg_align,
    moegg_dtype_t dtype, moegg_b_layout_t b_layout, int block_m, void* stream);

/*
 * The contiguous GEMM alone, driven by the tile list that an earlier
 * moegg_schedule or moegg_grouped_gemm_contiguous call left in `ws` (the
 * M-grouped contiguous layout of the DeepGEMM record, "Workarounds"; the
 * histogram and the choices made from it stay on the device, the padding
 * page's "Adapt kernels without adding a CPU stall").  One MoE layer runs
 * several grouped GEMMs over one routing histogram (gate/up, then down
 * projection); they can share one schedule.  Arguments are those of
 * moegg_grouped_gemm_contiguous, without m_sizes and seg_align.  The
 * schedule must come from the same G and rows_total.  block_m = 0 runs
 * whatever height the schedule used, in one launch whose grid depends only on
 * G, rows_total and N (so a captured graph stays valid when the counts and
 * the device's choice change between replays).  Any other block_m runs only
 * that height (MOEGG_BLOCK_M_PER_EXPERT: per-expert heights); if it differs
 * from the schedule's, nothing is written.
 */
moegg_status_t moegg_grouped_gemm_contiguous_scheduled(
    const void* A, const void* A_scale, const void* B, const void* B_scale, void* C,
    int G, int64_t rows_total, int K, int N, moegg_dtype_t dtype, moegg_b_layout_t b_layout,
    int block_m, const void* ws, size_t ws_bytes, void* stream);

/*
 * First expert projection with SwiGLU fused into its epilogue, for the
 * compute half of a fused MoE layer on one GPU (the DeepGEMM record's Mega
 * MoE fuses the expert GEMMs and SwiGLU so activations stay on chip; here
 * the gate and up products never reach HBM: only H does, once, in bf16).
 * Driven by the tile list an earlier moegg_schedule or
 * moegg_grouped_gemm_contiguous call left in `ws` (same G, rows_total).
 *   A        [rows_total, K] as for the contiguous call: bf16, e4m3 with
 *            fp32 1x128 scales ([rows_total, K/128], or [K/128, rows_total]
 *            with MOEGG_FP8_E4M3_SCALE_KM), or (MOEGG_FP8_E4M3_FP4_E2M1) e4m3
 *            with E8M0 scale bytes [K/128, rows_total].  MOEGG_FP8_E4M3_E8M0
 *            is not supported here.
 *   W1       [G, 2I, K] (K-contiguous: b_layout MOEGG_B_NK, or its
 *            256-row panels with MOEGG_B_NK_PANEL): for q = 0 .. I/16 - 1
 *            and w = 0 .. 15, row 32q + w is gate column 16q + w and row
 *            32q + 16 + w is up column 16q + w.  W1_scale (fp8): fp32
 *            [G, K/128, 2I/128] over those interleaved rows.
 *            MOEGG_FP8_E4M3_FP4_E2M1: packed E2M1 [G, 2I, K/2] (or its
 *            panels), same row order, E8M0 W1_scale bytes [G, K/128, 2I/128].
 *   H        [rows_total, I].  For each valid row R of expert e:
 *                g = sum_k A[R,k] Wgate_e[k,c],  u = sum_k A[R,k] Wup_e[k,c],
 *                h[R, c] = silu(g) * u,  silu(g) = g / (1 + e^-g)
 *            with fp32 accumulation and fp32 SwiGLU.  H_scale NULL: H is bf16,
 *            H[R, c] = bf16_rne(h).  H_scale set: H holds e4m3 codes and
 *            H_scale fp32 [rows_total, I/128] (MOEGG_FP8_E4M3_SCALE_KM:
 *            [I/128, rows_total]) one scale per 1x128 group, the input
 *            format of the fp8 contiguous call with the same dtype:
 *                s = amax over the group of |h| / 448 (1 if the amax is 0),
 *                H[R, c] = e4m3_rne(clamp(h / s, -448, 448)).
 *            Other rows untouched.
 * The down projection is then moegg_grouped_gemm_contiguous_scheduled on H
 * (K = I, with H_scale as its A_scale in the e4m3 case) from the same
 * schedule.  Constraints: those of the contiguous call with N = 2I, so
 * I % 128 == 0; H_scale 4-byte aligned.  block_m as in the scheduled call.
 */
moegg_status_t moegg_grouped_gemm_swiglu_scheduled(
    const void* A, const void* A_scale, const void* W1, const void* W1_scale, void* H, void* H_scale,
    int G, int64_t rows_total, int K, int I, moegg_dtype_t dtype, moegg_b_layout_t b_layout,
    int block_m, const void* ws, size_t ws_bytes, void* stream);

/*
 * Expert MLP in one launch: the SwiGLU projection and the down projection of
 * every expert in one kernel launch (the DeepGEMM record's "Arithmetic
 * intensity" section: Mega MoE fuses linear 1, SwiGLU and linear 2 so the
 * activations between them need not round-trip HBM; the dispatch and combine
 * it also fuses are inter-GPU and not part of this call).  It computes
 * exactly what moegg_grouped_gemm_contiguous with block_m = 256 (scheduler),
 * moegg_grouped_gemm_swiglu_scheduled (H = SwiGLU projection, e4m3 H with fp32
 * scales) and moegg_grouped_gemm_contiguous_scheduled on H compute in turn,
 * bit for bit, from one stream-ordered call:
 *   A        e4m3 [rows_total, K], A_scale fp32 [rows_total, K/128]
 *            (MOEGG_FP8_E4M3_SCALE_KM: [K/128, rows_total]).
 *   W1       e4m3 [G, 2I, K] with gate/up rows interleaved as for the SwiGLU
 *            call, W1_scale fp32 [G, K/128, 2I/128].
 *   W2       e4m3 [G, N2, I], W2_scale fp32 [G, I/128, N2/128].
 *            b_layout: MOEGG_B_NK for both weights, or MOEGG_B_NK_PANEL with
 *            P = 256 for both.
 *   H        e4m3 [rows_total, I], H_scale fp32 [rows_total, I/128]
 *            (SCALE_KM: [I/128, rows_total]): caller-owned intermediate,
 *            written and read back by the kernel; valid rows hold the SwiGLU
 *            call's output afterwards.
 *   Y        bf16 [rows_total, N2]: valid rows = H W2 per expert (fp32
 *            accumulation, one bf16 rounding); other rows untouched.
 *   m_sizes, G, rows_total, seg_align: as for the contiguous call (the tile
 *            list is always 256 rows tall).
 *   dtype    MOEGG_FP8_E4M3 or MOEGG_FP8_E4M3_SCALE_KM (else UNSUPPORTED).
 *   ws       moegg_workspace_bytes(G, rows_total), 256-byte aligned; also
 *            holds the row tiles' completion counters, which the call's
 *            scheduler launch clears.
 * Constraints: K % 128 == 0, I % 128 == 0, N2 % 256 == 0, every pointer
 * 16-byte aligned (scales 4).  One workgroup per tile, every SwiGLU tile
 * ahead of every down-projection tile in the grid; a row tile's
 * down-projection tiles wait (bounded) for all of its SwiGLU tiles.  A wait
 * that exceeds its bound sets MOEGG_FLAG_SYNC_TIMEOUT in the stats (the
 * affected Y rows are then unspecified); moegg_stats_read shows it.  Calls that
 * share ws must not overlap.
 */
moegg_status_t moegg_expert_mlp_fused(
    const void* A, const float* A_scale, const void* W1, const float* W1_scale, const void* W2,
    const float* W2_scale, void* H, float* H_scale, void* Y, const int32_t* m_sizes, int G,
    int64_t rows_total, int K, int I, int N2, int seg_align, moegg_dtype_t dtype,
    moegg_b_layout_t b_layout, void* ws, size_t ws_bytes, void* stream);

/*
 * Masked layout for decode under graph capture (DeepGEMM record,
 * "Workarounds" and "Arithmetic intensity": the kernel reads the per-expert
 * valid counts on the device and works on those rows only, so the token
 * counts never travel to the host).
 *   A        [G, cap, K].  A_scale fp32 [G, cap, K/128] (MOEGG_FP8_E4M3),
 *            fp32 [K/128, G * cap] (MOEGG_FP8_E4M3_SCALE_KM), E8M0
 *            bytes [K/128, G * cap] (MOEGG_FP8_E4M3_E8M0 and
 *            MOEGG_FP8_E4M3_FP4_E2M1; G * cap % 4 == 0), or NULL (bf16).
 *   B        as for the contiguous call.  B_scale as for the contiguous call.
 *   C        bf16 [G, cap, N].  Only rows r < masked_m[e] are written.
 *   masked_m int32 [G] on the device, read by the kernel at run time.
 * The grid depends only on G and N (one workgroup per expert and 128-column
 * tile, walking that expert's rows up to masked_m[e] in 128-row tiles, the
 * last one 64 or 128 rows tall), so a captured graph stays valid when
 * masked_m changes between replays.  Experts with masked_m[e] = 0 load no
 * weights.  ws may be NULL (no stats).  Otherwise stats are written as for
 * the contiguous call, with block_m = 128 and tiles = the sum of
 * ceil(masked_m[e] / 128).
 * Constraints: as for the contiguous call, plus cap >= 1.
 */
moegg_status_t moegg_grouped_gemm_masked(
    const void* A, const void* A_scale, const void* B, const void* B_scale, void* C,
    const int32_t* masked_m, int G, int cap, int K, int N,
    moegg_dtype_t dtype, moegg_b_layout_t b_layout,
    void* ws, size_t ws_bytes, void* stream);

/*
 * K-grouped weight gradient (DeepGEMM record, "Workarounds": MoE weight
 * backward with M and N fixed and the reduction axis grouped).
 *   X        bf16 [T, Mw], dY bf16 [T, Nw]: rows grouped by expert in expert
 *            order, t_sizes[e] rows each (device int32 [G]).
 *   dW       fp32 [G, Mw, Nw], overwritten:
 *                dW[e, i, j] = sum over expert e's rows t of X[t, i] * dY[t, j]
 *            with fp32 accumulation.  t_e = 0 writes zeros.
 * Experts are started longest first.  Constraints: Mw % 256 == 0,
 * Nw % 256 == 0, T >= 0; X and dY may be NULL when T = 0.  A workspace is
 * required (expert offsets and order).
 */
moegg_status_t moegg_grouped_gemm_k_grouped(
    const void* X, const void* dY, float* dW, const int32_t* t_sizes, int G, int64_t T,
    int Mw, int Nw, void* ws, size_t ws_bytes, void* stream);

/*
 * K-grouped weight gradient on e4m3 operands with fp32 scales (DeepGEMM
 * record, "Workarounds": the K-grouped MoE weight backward next to FP8 with
 * per-group scaling).  The scale groups lie along the reduction (token) axis:
 * one group is up to 128 consecutive rows of one expert's segment, counted
 * from the segment's first row, so groups restart at every segment start and
 * the last group of a segment may be short.  Groups are numbered across
 * experts in order: expert e's first group is
 *     goff[e] = sum_{j<e} ceil(t_j / 128)
 * (over the counts as used: negative counts read as 0, segments truncated at
 * T).  Each scale covers one column over one group.
 *   X         e4m3 [T, Mw], dY e4m3 [T, Nw]: rows grouped by expert in expert
 *             order, t_sizes[e] rows each (device int32 [G]).
 *   X_scale   fp32 [scale_groups, Mw]; row g scales X's columns over group g.
 *   dY_scale  fp32 [scale_groups, Nw]; likewise for dY.
 *   dW        fp32 [G, Mw, Nw], overwritten:
 *               dW[e, i, j] = sum over expert e's rows t of
 *                   (X[t, i] * X_scale[g(t), i]) * (dY[t, j] * dY_scale[g(t), j])
 *             with g(t) = goff[e] + (t - first row of e) / 128.  Each group's
 *             fp32 partial sum of code products is multiplied by its two
 *             scales and added to the fp32 accumulator.  t_e = 0 writes zeros.
 *   scale_groups  rows of the scale arrays, at least sum_e ceil(t_e / 128)
 *             (at most T / 128 + G).  A histogram that needs more sets
 *             MOEGG_FLAG_SCALE_GROUPS; the missing groups' scales read as 0.
 * Experts are started longest first.  Constraints: as for
 * moegg_grouped_gemm_k_grouped; scale arrays 4-byte aligned, and
 * scale_groups * max(Mw, Nw) * 4 < 2^31 (UNSUPPORTED otherwise).
 */
moegg_status_t moegg_grouped_gemm_k_grouped_fp8(
    const void* X, const float* X_scale, const void* dY, const float* dY_scale, float* dW,
    const int32_t* t_sizes, int G, int64_t T, int Mw, int Nw, int64_t scale_groups,
    void* ws, size_t ws_bytes, void* stream);

/*
 * K-grouped weight gradient on e4m3 operands with E8M0 scales (DeepGEMM
 * record, "Workarounds": the K-grouped MoE weight backward; the same record
 * lists packed UE8M0 scale factors as the newer architecture's format).  The
 * groups are those of moegg_grouped_gemm_k_grouped_fp8; each scale is an
 * exponent byte b meaning 2^(b - 127).
 *   X_scale   uint8 [scale_groups, Mw]; row g scales X's columns over group g.
 *   dY_scale  uint8 [scale_groups, Nw]; likewise for dY.
 *   dW        fp32 [G, Mw, Nw], overwritten:
 *               dW[e, i, j] = sum over expert e's rows t of
 *                   (X[t, i] * 2^(X_scale[g(t), i] - 127)) * (dY[t, j] * 2^(dY_scale[g(t), j] - 127))
 *             in fp32.  The scales scale exactly (powers of two), so the
 *             MFMA applies them to each group's products and accumulates
 *             the group into dW's accumulator directly.  t_e = 0 writes zeros.
 *   scale_groups  as for moegg_grouped_gemm_k_grouped_fp8.  A histogram that
 *             needs more sets MOEGG_FLAG_SCALE_GROUPS; the missing groups'
 *             scale bytes read as 0 (2^-127), which flushes their products to
 *             zero.
 * Constraints: as for moegg_grouped_gemm_k_grouped; scale arrays 4-byte
 * aligned, and scale_groups * max(Mw, Nw) < 2^31 (UNSUPPORTED otherwise).
 */
moegg_status_t moegg_grouped_gemm_k_grouped_e8m0(
    const void* X, const uint8_t* X_scale, const void* dY, const uint8_t* dY_scale, float* dW,
    const int32_t* t_sizes, int G, int64_t T, int Mw, int Nw, int64_t scale_groups,
    void* ws, size_t ws_bytes, void* stream);

/* Copy the stats of the last scheduled call on `ws` to the host.
 * Synchronizes `stream`. */
moegg_status_t moegg_stats_read(const void* ws, moegg_stats_t* h_out, void* stream);

/* Copy up to cap_tiles tile-list entries to h_tiles, and the entry count to
 * *h_n.  Synchronizes `stream`. */
moegg_status_t moegg_tile_list_read(const void* ws, moegg_tile_t* h_tiles, int64_t cap_tiles,
                                    int64_t* h_n, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOEGG_H */
