/*
 * oracle.c -- plain, slow fp64 CPU reference for the MoE grouped GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this file's library.  The HIP
 * product path never calls it, and the two share no code.
 *
 * What it computes, from the pages:
 *   - Grouping routes each expert's tokens into one GEMM; it alters how the
 *     work is tiled, while every output stays the same product (DeepGEMM
 *     grouped/masked MoE GEMM record, "Arithmetic intensity").  Each expert e multiplies its
 *     own routed rows by its own weight, and all experts share K and N.  So
 *     every valid output element is the plain dot product
 *         C[row, n] = sum_k A[row, k] * B_e[k, n]
 *     summed here in fp64, k ascending, one output row at a time.
 *   - The three layouts named under "Workarounds" of the same record:
 *     M-grouped contiguous, masked (capacity buffer plus valid counts), and
 *     K-grouped for the weight gradient (dW_e = X_e^T dY_e).
 *   - FP8 with per-group fp32 scales ("Workarounds").  Each element is decoded
 *     and multiplied by its group's scale before the product:
 *         A[row, k] = dec(qa) * a_s[row, k/128]
 *         B_e[k, n] = dec(qb) * b_s[e, k/128, n/128]
 *
 * Decoders are written from the format definitions:
 *   - bf16 = the top 16 bits of an IEEE binary32.
 *   - OCP e4m3fn = 1 sign, 4 exponent (bias 7), 3 mantissa bits.  Subnormals
 *     at exponent 0.  S.1111.111 is NaN.  No infinities.
 *
 * The loop order for each output row is k outer, n inner, with an fp64
 * accumulator per n.  Every output element is still summed over k in
 * ascending order, exactly as the definition reads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_BF16 = 0, ORC_FP8 = 1 };       /* operand storage type            */
enum { ORC_B_KN = 0, ORC_B_NK = 1 };      /* B_e stored [K,N] or [N,K]       */
#define ORC_GROUP 128                     /* fp8 scale group along K and N   */

double oracle_dec_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_dec_e4m3(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);          /* subnormal: m/8 * 2^-6 */
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);        /* normal: 1.m * 2^(e-7) */
    return s ? -v : v;
}

/* A element (row-major [rows, K]), scaled when fp8. */
static double a_elem(int dtype, const void* A, const float* As, int64_t row, int K, int k) {
    if (dtype == ORC_BF16) return oracle_dec_bf16(((const uint16_t*)A)[row * K + k]);
    return oracle_dec_e4m3(((const uint8_t*)A)[row * K + k]) *
           (double)As[row * (K / ORC_GROUP) + k / ORC_GROUP];
}

/* B_e element at (k, n), scaled when fp8.  Scales are [G, K/128, N/128]. */
static double b_elem(int dtype, int layout, const void* B, const float* Bs,
                     int e, int K, int N, int k, int n) {
    int64_t idx = layout == ORC_B_KN ? ((int64_t)e * K + k) * N + n
                                     : ((int64_t)e * N + n) * K + k;
    if (dtype == ORC_BF16) return oracle_dec_bf16(((const uint16_t*)B)[idx]);
    return oracle_dec_e4m3(((const uint8_t*)B)[idx]) *
           (double)Bs[((int64_t)e * (K / ORC_GROUP) + k / ORC_GROUP) * (N / ORC_GROUP) + n / ORC_GROUP];
}

/* One output row: out[n] = sum_k A[arow, k] * B_e[k, n]. */
static void row_product(int dtype, int layout, const void* A, const float* As, int64_t arow,
                        const void* B, const float* Bs, int e, int K, int N, double* out) {
    for (int n = 0; n < N; ++n) out[n] = 0.0;
    for (int k = 0; k < K; ++k) {
        double a = a_elem(dtype, A, As, arow, K, k);
        for (int n = 0; n < N; ++n) out[n] += a * b_elem(dtype, layout, B, Bs, e, K, N, k, n);
    }
}

/*
 * M-grouped contiguous layout.  Expert e's m_e rows start at
 *     seg_off[e] = sum_{j<e} align_up(m_j, seg_align)
 * in A[rows_total, K] and C[rows_total, N].  For each requested row index,
 * out[i, :] receives that row of C, or NaN if the row belongs to no expert.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_contiguous(int dtype, int layout, const void* A, const float* As,
                      const void* B, const float* Bs, const int32_t* m_sizes, int G,
                      int64_t rows_total, int K, int N, int seg_align,
                      const int64_t* rows, int64_t nrows, double* out) {
    if (G <= 0 || K <= 0 || N <= 0 || seg_align <= 0) return -1;
    if (dtype == ORC_FP8 && (K % ORC_GROUP || N % ORC_GROUP)) return -1;
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
    if (!off) return -1;
    off[0] = 0;
    for (int e = 0; e < G; ++e) {
        int64_t m = m_sizes[e];
        off[e + 1] = off[e] + (m + seg_align - 1) / seg_align * seg_align;
    }
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        double* o = out + i * (int64_t)N;
        int e_found = -1;
        for (int e = 0; e < G; ++e)
            if (r >= off[e] && r < off[e] + m_sizes[e]) { e_found = e; break; }
        if (e_found < 0 || r >= rows_total) {
            for (int n = 0; n < N; ++n) o[n] = NAN;
            if (r < 0 || r >= rows_total) bad = 1;
            continue;
        }
        row_product(dtype, layout, A, As, r, B, Bs, e_found, K, N, o);
    }
    free(off);
    return bad ? -1 : 0;
}

/*
 * Masked layout: A[G, cap, K], C[G, cap, N]; expert e's valid rows are
 * r < masked_m[e] (at most cap).  Each request (experts[i], rs[i]) gets
 * C[e, r, :], or NaN when r is not a valid row of e.
 */
int oracle_masked(int dtype, int layout, const void* A, const float* As,
                  const void* B, const float* Bs, const int32_t* masked_m, int G, int cap,
                  int K, int N, const int32_t* experts, const int32_t* rs, int64_t nreq,
                  double* out) {
    if (G <= 0 || cap <= 0 || K <= 0 || N <= 0) return -1;
    if (dtype == ORC_FP8 && (K % ORC_GROUP || N % ORC_GROUP)) return -1;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < nreq; ++i) {
        int e = experts[i], r = rs[i];
        double* o = out + i * (int64_t)N;
        if (e < 0 || e >= G || r < 0 || r >= cap) { bad = 1; continue; }
        if (r >= masked_m[e]) {
            for (int n = 0; n < N; ++n) o[n] = NAN;
            continue;
        }
        row_product(dtype, layout, A, As, (int64_t)e * cap + r, B, Bs, e, K, N, o);
    }
    return bad ? -1 : 0;
}

/*
 * K-grouped weight gradient: the rows of X[T, Mw] and dY[T, Nw] are grouped
 * by expert in order, t_sizes[e] rows each.  The reduction runs over each
 * expert's own rows:
 *     dW[e, i, j] = sum_{t in expert e's rows} X[t, i] * dY[t, j]
 * An expert with no rows gets the empty sum, 0.  Each request
 * (experts[i], is[i]) gets the dW row dW[e, i, :].
 */
int oracle_k_grouped(const uint16_t* X, const uint16_t* dY, const int32_t* t_sizes, int G,
                     int64_t T, int Mw, int Nw, const int32_t* experts, const int32_t* is,
                     int64_t nreq, double* out) {
    if (G <= 0 || Mw <= 0 || Nw <= 0) return -1;
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
    if (!off) return -1;
    off[0] = 0;
    for (int e = 0; e < G; ++e) off[e + 1] = off[e] + t_sizes[e];
    if (off[G] > T) { free(off); return -1; }
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t q = 0; q < nreq; ++q) {
        int e = experts[q], i = is[q];
        double* o = out + q * (int64_t)Nw;
        if (e < 0 || e >= G || i < 0 || i >= Mw) { bad = 1; continue; }
        for (int j = 0; j < Nw; ++j) o[j] = 0.0;
        for (int64_t t = off[e]; t < off[e + 1]; ++t) {
            double x = oracle_dec_bf16(X[t * Mw + i]);
            for (int j = 0; j < Nw; ++j) o[j] += x * oracle_dec_bf16(dY[t * Nw + j]);
        }
    }
    free(off);
    return bad ? -1 : 0;
}

/*
 * K-grouped weight gradient with e4m3 operands and fp32 scales along the
 * reduction axis (DeepGEMM record, "Workarounds": the K-grouped MoE weight
 * backward next to FP8 with per-group scaling).  The reduction axis is the
 * token axis, so each scale group is 128 consecutive rows of one expert's
 * segment and one column:
 *   - expert e's segment starts at off[e] = sum_{j<e} t_j and holds t_e rows;
 *   - its groups are its rows 0..127, 128..255, ... counted from the segment
 *     start (the last group may hold fewer than 128 rows);
 *   - groups are numbered across experts in order: expert e's first group is
 *     goff[e] = sum_{j<e} ceil(t_j / 128);
 *   - Xs[g, i] scales column i of X in group g, dYs[g, j] column j of dY.
 * Then
 *     dW[e, i, j] = sum over expert e's rows t of
 *                   (dec(X[t, i]) * Xs[g(t), i]) * (dec(dY[t, j]) * dYs[g(t), j])
 * with g(t) = goff[e] + (t - off[e]) / 128, summed in fp64, t ascending.
 * Xs is [n_groups, Mw] and dYs [n_groups, Nw]; n_groups must cover every
 * group.  An expert with no rows gets 0.  Each request (experts[i], is[i])
 * gets the dW row dW[e, i, :].
 */
int oracle_k_grouped_fp8(const uint8_t* X, const float* Xs, const uint8_t* dY, const float* dYs,
                         const int32_t* t_sizes, int G, int64_t T, int Mw, int Nw, int64_t n_groups,
                         const int32_t* experts, const int32_t* is, int64_t nreq, double* out) {
    if (G <= 0 || Mw <= 0 || Nw <= 0 || n_groups < 0) return -1;
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
    int64_t* goff = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
    if (!off || !goff) { free(off); free(goff); return -1; }
    off[0] = 0;
    goff[0] = 0;
    for (int e = 0; e < G; ++e) {
        if (t_sizes[e] < 0) { free(off); free(goff); return -1; }
        off[e + 1] = off[e] + t_sizes[e];
        goff[e + 1] = goff[e] + (t_sizes[e] + 127) / 128;
    }
    if (off[G] > T || goff[G] > n_groups) { free(off); free(goff); return -1; }
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t q = 0; q < nreq; ++q) {
        int e = experts[q], i = is[q];
        double* o = out + q * (int64_t)Nw;
        if (e < 0 || e >= G || i < 0 || i >= Mw) { bad = 1; continue; }
        for (int j = 0; j < Nw; ++j) o[j] = 0.0;
        for (int64_t t = off[e]; t < off[e + 1]; ++t) {
            int64_t g = goff[e] + (t - off[e]) / 128;
            double x = oracle_dec_e4m3(X[t * Mw + i]) * (double)Xs[g * Mw + i];
            for (int j = 0; j < Nw; ++j)
                o[j] += x * (oracle_dec_e4m3(dY[t * Nw + j]) * (double)dYs[g * Nw + j]);
        }
    }
    free(off);
    free(goff);
    return bad ? -1 : 0;
}

/* Number of OpenMP threads a parallel region uses (1 without OpenMP). */
int oracle_threads(void) {
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
