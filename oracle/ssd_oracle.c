/*
 * ssd_oracle.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, fp64 CPU evaluation of the selective state space model with a
 * scalar decay per head (the Mamba-2 "SSD" layer), written as the sequential
 * recurrence it is defined by.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP library under mamba_ssd_scan_02_amd/.
 *
 * What is computed, and where it comes from:
 *
 *  - The discrete recurrence h_t = Abar h_{t-1} + Bbar x_t with zero-order-hold
 *    Abar = exp(Delta A) and Bbar ~= Delta B: page "State Space Model"
 *    (book.paithon.it), section "Un sistema che riassume il passato", the
 *    paragraph on discretisation; page "State Space Models (SSM)"
 *    (ultralytics.com glossary), section "Come funzionano gli SSM".
 *  - The transition is one scalar per step, Abar_t = a_t I (every state entry
 *    fades at the same rate): page "State Space Model", sections
 *    "Due strade, una meta" and "Da ricordare".
 *  - The read-out y = C h + D x: page "Puntata 205 -- State Space Models e
 *    Mamba" (aiperbabbani.it), section "Cos'e' un SSM, in 30 secondi".
 *  - Delta, B and C change with every token (selectivity): same page, section
 *    "Mamba (Gu & Dao, dicembre 2023): selective scan".
 *  - Each input channel drives its own row of N state entries, read together
 *    by C: page "State Space Model", section "Un sistema che riassume il
 *    passato" (the row of tanks per channel).  So the per-head state is P x N.
 *  - Heads share B and C within a group; head h uses group h / (H / G).  The
 *    pages say nothing about groups: this is the plainest contiguous reading.
 *
 * Order inside one step (the state is updated first, then read out, so the
 * current input reaches y_t with weight 1, as in the water-tank example where
 * the level right after the first pour is 2):
 *     a          = exp(dt[b,t,h] * A[h])
 *     S[p][n]    = a * S[p][n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *     y[b,t,h,p] = sum_n C[b,t,g,n] * S[p][n] + D[h] * x[b,t,h,p]
 *
 * Two discretisations of the input term (the `zoh` flag of the _ex calls):
 *   0  Bbar = Delta B, the first-order form the selective scan uses (page
 *      "State Space Model", section "Un sistema che riassume il passato");
 *   1  the exact zero-order hold Bbar = (Abar - 1) / A B, i.e. the input weight
 *      expm1(Delta A) / A in place of Delta (Delta itself where A = 0), as in
 *      the demonstration of the recurrent and convolutional forms on page
 *      "State Space Models (SSM)" (ultralytics.com glossary), section "Come
 *      funzionano gli SSM".
 *
 * Inputs are read in their storage type (fp32, or bf16 bit patterns widened
 * exactly) and every operation after that is fp64 with libm exp() and
 * expm1().  Compile without -ffast-math.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_IN_F32 0
#define ORACLE_IN_BF16 1

/* Widen one stored element to double.  bf16 is the upper half of an IEEE
 * binary32, so shifting its bits up by 16 gives the same number exactly. */
static double widen(const void* base, int32_t kind, int64_t i) {
    if (kind == ORACLE_IN_F32) return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int32_t oracle_abi_version(void) { return 2; }

/* Weight of the input term for one step: Delta, or the zero-order-hold
 * (exp(Delta A) - 1) / A (Delta where A = 0). */
static double input_weight(double d, double Ah, int32_t zoh) {
    if (!zoh || Ah == 0.0) return d;
    return expm1(d * Ah) / Ah;
}

/* Threads an OpenMP parallel region of this library will use. */
int32_t oracle_max_threads(void) {
    int32_t n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = (int32_t)omp_get_num_threads();
    }
    return n;
}

/*
 * Whole-sequence forward for a list of (batch, head) pairs.
 *
 *   x   [batch][L][H][P]   kind in_kind        dt [batch][L][H] fp32 (already Delta)
 *   A   [H] fp32                               D  [H] fp32, may be NULL (no skip term)
 *   Bm  [batch][L][G][N]   kind in_kind        Cm [batch][L][G][N] kind in_kind
 *   init[batch][H][P][N] fp32, may be NULL (empty state)
 *   bh  [n_bh][2] = (b, h) pairs to evaluate
 *   y_sel     [n_bh][L][P] fp64 output (may be NULL)
 *   final_sel [n_bh][P][N] fp64 output (may be NULL)
 *   t_begin, t_end: only tokens t in [t_begin, t_end) are written to y_sel
 *                   (row t - t_begin); the recurrence still runs from t = 0.
 *                   Pass 0 and L for the whole sequence.
 * Returns 0, or a negative number for a bad argument.
 */
int32_t oracle_ssd_forward_ex(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                              int64_t G, int32_t in_kind, const void* x, const float* dt,
                              const float* A, const void* Bm, const void* Cm, const float* D,
                              const float* init, const int64_t* bh, int64_t n_bh, int64_t t_begin,
                              int64_t t_end, double* y_sel, double* final_sel, int32_t zoh) {
    if (batch < 1 || L < 0 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return -1;
    if (!x || !dt || !A || !Bm || !Cm || !bh || n_bh < 0) return -2;
    if (t_begin < 0 || t_end > L || t_begin > t_end) return -3;
    const int64_t heads_per_group = H / G;
    int32_t bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t k = 0; k < n_bh; ++k) {
        const int64_t b = bh[2 * k], h = bh[2 * k + 1];
        if (b < 0 || b >= batch || h < 0 || h >= H) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        const int64_t g = h / heads_per_group;
        double* S = (double*)malloc((size_t)(P * N) * sizeof(double));
        double* xr = (double*)malloc((size_t)P * sizeof(double));
        double* br = (double*)malloc((size_t)N * sizeof(double));
        double* cr = (double*)malloc((size_t)N * sizeof(double));
        for (int64_t e = 0; e < P * N; ++e)
            S[e] = init ? (double)init[((b * H + h) * P) * N + e] : 0.0;
        const double Ah = (double)A[h];
        const double Dh = D ? (double)D[h] : 0.0;

        for (int64_t t = 0; t < L; ++t) {
            const double d = (double)dt[(b * L + t) * H + h];
            const double a = exp(d * Ah);
            const double w = input_weight(d, Ah, zoh);
            for (int64_t p = 0; p < P; ++p) xr[p] = widen(x, in_kind, ((b * L + t) * H + h) * P + p);
            for (int64_t n = 0; n < N; ++n) {
                br[n] = widen(Bm, in_kind, ((b * L + t) * G + g) * N + n);
                cr[n] = widen(Cm, in_kind, ((b * L + t) * G + g) * N + n);
            }
            /* state update: S <- a S + w * x (outer) B, w = dt or the ZOH weight */
            for (int64_t p = 0; p < P; ++p) {
                const double u = w * xr[p];
                double* row = S + p * N;
                for (int64_t n = 0; n < N; ++n) row[n] = a * row[n] + u * br[n];
            }
            /* read-out: y = C . S + D x */
            if (y_sel && t >= t_begin && t < t_end) {
                double* yrow = y_sel + (k * (t_end - t_begin) + (t - t_begin)) * P;
                for (int64_t p = 0; p < P; ++p) {
                    const double* row = S + p * N;
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) acc += cr[n] * row[n];
                    yrow[p] = acc + Dh * xr[p];
                }
            }
        }
        if (final_sel) memcpy(final_sel + k * P * N, S, (size_t)(P * N) * sizeof(double));
        free(S);
        free(xr);
        free(br);
        free(cr);
    }
    return bad ? -4 : 0;
}

int32_t oracle_ssd_forward(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                           int32_t in_kind, const void* x, const float* dt, const float* A,
                           const void* Bm, const void* Cm, const float* D, const float* init,
                           const int64_t* bh, int64_t n_bh, int64_t t_begin, int64_t t_end,
                           double* y_sel, double* final_sel) {
    return oracle_ssd_forward_ex(batch, L, H, P, N, G, in_kind, x, dt, A, Bm, Cm, D, init, bh,
                                 n_bh, t_begin, t_end, y_sel, final_sel, 0);
}

/*
 * One decode step for every (batch, head): the same update and read-out as a
 * single iteration of the loop above, on a caller-held fp64 state.  This is the
 * step-by-step way of running the model that the pages say is used to generate
 * (page "State Space Model", section "Un sistema che riassume il passato", the
 * last part of the water-tank passage).
 *
 *   state [batch][H][P][N] fp64, updated in place
 *   x_t   [batch][H][P] kind in_kind     dt_t [batch][H] fp32
 *   B_t, C_t [batch][G][N] kind in_kind  A, D [H] fp32 (D may be NULL)
 *   y_t   [batch][H][P] fp64 output
 */
int32_t oracle_ssm_step_ex(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G,
                           int32_t in_kind, double* state, const void* x_t, const float* dt_t,
                           const float* A, const void* B_t, const void* C_t, const float* D,
                           double* y_t, int32_t zoh) {
    if (batch < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return -1;
    if (!state || !x_t || !dt_t || !A || !B_t || !C_t || !y_t) return -2;
    const int64_t heads_per_group = H / G;

#pragma omp parallel for schedule(static)
    for (int64_t bhi = 0; bhi < batch * H; ++bhi) {
        const int64_t b = bhi / H, h = bhi % H, g = h / heads_per_group;
        const double d = (double)dt_t[b * H + h];
        const double a = exp(d * (double)A[h]);
        const double w = input_weight(d, (double)A[h], zoh);
        const double Dh = D ? (double)D[h] : 0.0;
        double* S = state + bhi * P * N;
        for (int64_t p = 0; p < P; ++p) {
            const double xp = widen(x_t, in_kind, bhi * P + p);
            const double u = w * xp;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double bn = widen(B_t, in_kind, (b * G + g) * N + n);
                const double cn = widen(C_t, in_kind, (b * G + g) * N + n);
                S[p * N + n] = a * S[p * N + n] + u * bn;
                acc += cn * S[p * N + n];
            }
            y_t[bhi * P + p] = acc + Dh * xp;
        }
    }
    return 0;
}

int32_t oracle_ssm_step(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G, int32_t in_kind,
                        double* state, const void* x_t, const float* dt_t, const float* A,
                        const void* B_t, const void* C_t, const float* D, double* y_t) {
    return oracle_ssm_step_ex(batch, H, P, N, G, in_kind, state, x_t, dt_t, A, B_t, C_t, D, y_t, 0);
}
