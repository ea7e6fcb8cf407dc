/* Host-side checks run under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built and run by tests/test_sanitize_host.py), as two programs:
 *   - CHECK_LIBRARY: the library's argument checking.  Every call here fails
 *     before any launch, so no GPU is needed, and each must return the
 *     documented code;
 *   - CHECK_ORACLE: the fp64 oracle on small inputs.  A whole-sequence
 *     forward must leave the same final state and outputs as the same tokens
 *     fed one decode step at a time (both recurrences walk the same update),
 *     for fp32 and bf16 inputs and for both discretisations.
 * Pointers passed to the library are distinct fake device addresses: the
 * checks only compare them, never dereference them. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#ifdef CHECK_LIBRARY
#include "ssd_mi355x.h"
#endif

int32_t oracle_ssd_forward_ex(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                              int64_t G, int32_t in_kind, const void* x, const float* dt,
                              const float* A, const void* Bm, const void* Cm, const float* D,
                              const float* init, const int64_t* bh, int64_t n_bh, int64_t t_begin,
                              int64_t t_end, double* y_sel, double* final_sel, int32_t zoh);
int32_t oracle_ssm_step_ex(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G,
                           int32_t in_kind, double* state, const void* x_t, const float* dt_t,
                           const float* A, const void* B_t, const void* C_t, const float* D,
                           double* y_t, int32_t zoh);

static int fails = 0;
#define CHECK(cond)                                              \
    do {                                                         \
        if (!(cond)) {                                           \
            printf("FAIL line %d: %s\n", __LINE__, #cond);       \
            ++fails;                                             \
        }                                                        \
    } while (0)

#ifdef CHECK_LIBRARY
/* fake device addresses, 256 MiB apart */
#define FAKE(i) ((void*)(uintptr_t)(0x100000000ull + (uint64_t)(i) * 0x10000000ull))

static void library_checks(void) {
    const int64_t b = 1, L = 64, H = 2, P = 16, N = 16, G = 1, Q = 64;
    void *x = FAKE(1), *B = FAKE(2), *C = FAKE(3), *y = FAKE(4), *ws = FAKE(5);
    float *dt = (float*)FAKE(6), *A = (float*)FAKE(7), *D = (float*)FAKE(8);
    float *init = (float*)FAKE(9), *fin = (float*)FAKE(10);
    const size_t need = ssd_forward_workspace_bytes(b, L, H, P, N, G, Q, SSD_DTYPE_F32);
    const int32_t f32 = SSD_DTYPE_F32;

    CHECK(ssd_abi_version() == SSD_ABI_VERSION);
    for (int32_t s = -3; s < 12; ++s) CHECK(ssd_status_str(s) != NULL && strlen(ssd_status_str(s)) > 0);

    /* workspace sizes: valid, invalid and overflowing */
    CHECK(need > 0);
    CHECK(ssd_forward_workspace_bytes(0, L, H, P, N, G, Q, f32) == 0);
    CHECK(ssd_forward_workspace_bytes(b, L, 3, P, N, 2, Q, f32) == 0);
    CHECK(ssd_forward_workspace_bytes(b, L, H, P, N, G, Q, 9) == 0);
    CHECK(ssd_forward_workspace_bytes(INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX, 1, 1, f32) == 0);
    CHECK(ssd_forward_workspace_bytes(1 << 24, 1 << 30, 65536, 128, 128, 1, 1, f32) == 0);
    CHECK(ssd_forward_workspace_bytes(b, L, H, P, N, G, INT64_MAX, f32) == 0);
    CHECK(ssd_forward_workspace_bytes(b, L, H, INT64_MAX, N, G, Q, f32) == 0);
    CHECK(ssd_forward_workspace_bytes(-1, -1, -1, -1, -1, -1, -1, f32) == 0);
    CHECK(ssd_state_passing_seg_workspace_bytes(1, 32, 64, 128, 64) > 0);
    CHECK(ssd_state_passing_seg_workspace_bytes(INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX, 2) == 0);

    /* forward: shape, dtype, NULL, workspace, alignment and alias errors */
    CHECK(ssd_forward(0, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_forward(b, L, 3, P, N, 2, Q, f32, x, dt, A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_forward(b, INT64_MAX, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, 9, x, dt, A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_UNSUPPORTED);
    CHECK(ssd_forward(b, L, H, 4096, N, G, Q, f32, x, dt, A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_UNSUPPORTED);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, NULL, dt, A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_NULL);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, NULL, A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_NULL);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, NULL, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_NULL);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, NULL, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_NULL);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, NULL, D, init, y, fin, ws, need, NULL) == SSD_ERR_NULL);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, NULL, fin, ws, need, NULL) == SSD_ERR_NULL);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, fin, NULL, need, NULL) == SSD_ERR_WORKSPACE);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, fin, ws, need - 1, NULL) == SSD_ERR_WORKSPACE);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, (char*)x + 4, dt, A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_ALIGN);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, (float*)((char*)dt + 2), A, B, C, D, init, y, fin, ws, need, NULL) == SSD_ERR_ALIGN);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, x, fin, ws, need, NULL) == SSD_ERR_ALIAS);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, (char*)B + 256, fin, ws, need, NULL) == SSD_ERR_ALIAS);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, (float*)x, ws, need, NULL) == SSD_ERR_ALIAS);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, (float*)D, ws, need, NULL) == SSD_ERR_ALIAS);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, fin, (char*)y + 512, need, NULL) == SSD_ERR_ALIAS);
    CHECK(ssd_forward(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, fin, A, need, NULL) == SSD_ERR_ALIAS);
    CHECK(ssd_forward_zoh(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, x, fin, ws, need, NULL) == SSD_ERR_ALIAS);
    /* the gated forward: z is an input like x */
    void* zz = FAKE(11);
    CHECK(ssd_forward_gated(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, NULL, y, fin, ws, need, NULL) == SSD_ERR_NULL);
    CHECK(ssd_forward_gated(0, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, NULL, y, fin, ws, need, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_forward_gated(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, y, fin, ws, need, NULL) == SSD_ERR_ALIAS);
    CHECK(ssd_forward_gated(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, zz, y, fin, (char*)zz + 256, need, NULL) == SSD_ERR_ALIAS);
    CHECK(ssd_forward_gated(b, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, (char*)zz + 4, y, fin, ws, need, NULL) == SSD_ERR_ALIGN);

    /* the allocation-free forward: sizes beyond its array are rejected first */
    CHECK(ssd_forward_noalloc(4, 8192, 80, 64, 128, 1, 256, SSD_DTYPE_BF16, x, dt, A, B, C, D, init, y, fin, NULL) == SSD_ERR_WORKSPACE);
    CHECK(ssd_forward_noalloc(b, L, H, P, N, G, Q, f32, NULL, dt, A, B, C, D, init, y, fin, NULL) == SSD_ERR_NULL);
    CHECK(ssd_forward_noalloc(0, L, H, P, N, G, Q, f32, x, dt, A, B, C, D, init, y, fin, NULL) == SSD_ERR_SHAPE);

    /* decode step */
    CHECK(ssm_step(0, H, P, N, G, f32, fin, x, dt, A, B, C, D, y, NULL) == SSD_ERR_SHAPE);
    CHECK(ssm_step(b, H, P, N, G, f32, NULL, x, dt, A, B, C, D, y, NULL) == SSD_ERR_NULL);
    CHECK(ssm_step(b, H, P, N, G, 7, fin, x, dt, A, B, C, D, y, NULL) == SSD_ERR_UNSUPPORTED);
    CHECK(ssm_step_zoh(b, 3, P, N, 2, f32, fin, x, dt, A, B, C, D, y, NULL) == SSD_ERR_SHAPE);

    /* stage calls */
    CHECK(ssd_chunk_cumsum(0, L, H, Q, dt, A, (float*)ws, (float*)y, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_chunk_cumsum(b, L, H, Q, NULL, A, (float*)ws, (float*)y, NULL) == SSD_ERR_NULL);
    CHECK(ssd_chunk_cumsum_zoh(b, L, H, Q, dt, A, NULL, (float*)y, NULL) == SSD_ERR_NULL);
    CHECK(ssd_chunk_state(b, L, H, P, N, G, Q, f32, NULL, B, dt, A, ws, NULL) == SSD_ERR_NULL);
    CHECK(ssd_chunk_state(b, L, H, P, N, G, Q, 9, x, B, dt, A, ws, NULL) == SSD_ERR_UNSUPPORTED);
    CHECK(ssd_chunk_cumsum_state(b, L, H, P, N, G, Q, f32, x, B, NULL, A, (float*)ws, (float*)y, C, NULL) == SSD_ERR_NULL);
    CHECK(ssd_chunk_cumsum_state(b, L, 3, P, N, 2, Q, f32, x, B, dt, A, (float*)ws, (float*)y, C, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_state_passing(b, L, H, P, N, Q, f32, NULL, dt, init, y, fin, NULL) == SSD_ERR_NULL);
    CHECK(ssd_state_passing(b, 0, H, P, N, Q, f32, ws, dt, init, y, fin, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_state_passing_seg(b, L, H, P, N, Q, 2, f32, ws, dt, init, y, fin, NULL, 0, NULL) == SSD_ERR_WORKSPACE);
    CHECK(ssd_state_scan(b, L, H, P, N, G, Q, f32, x, B, dt, A, init, y, fin, NULL) == SSD_ERR_UNSUPPORTED);
    CHECK(ssd_state_scan(b, 512, 2, 64, 128, 1, 256, SSD_DTYPE_BF16, NULL, B, dt, A, init, y, fin, NULL) == SSD_ERR_NULL);
    CHECK(ssd_chunk_scan(b, L, H, P, N, G, Q, f32, x, B, C, dt, A, NULL, D, y, NULL) == SSD_ERR_NULL);
    CHECK(ssd_chunk_scan(b, L, 3, P, N, 2, Q, f32, x, B, C, dt, A, ws, D, y, NULL) == SSD_ERR_SHAPE);

    /* the two-level stage calls and the forward's run length (no launch: every
       call below fails a check first) */
    const int32_t bf = SSD_DTYPE_BF16;
    CHECK(ssd_forward_run_chunks(b, L, H, P, N, G, Q, f32) == 0);
    CHECK(ssd_forward_run_chunks(INT64_MAX, INT64_MAX, INT64_MAX, 64, 128, 1, 256, bf) == 0);
    CHECK(ssd_forward_run_chunks(-1, -1, -1, -1, -1, -1, -1, bf) == 0);
    CHECK(ssd_chunk_state_runs(b, L, H, P, N, G, Q, f32, 2, x, B, dt, A, (float*)ws, (float*)y, C, (float*)D, (float*)init, NULL) == SSD_ERR_UNSUPPORTED);
    CHECK(ssd_chunk_state_runs(1, 512, 2, 64, 128, 1, 256, bf, 0, x, B, dt, A, (float*)ws, (float*)y, C, (float*)D, (float*)init, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_chunk_state_runs(1, 512, 2, 64, 128, 1, 256, bf, INT64_MAX, x, B, dt, A, (float*)ws, (float*)y, C, (float*)D, (float*)init, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_chunk_state_runs(1, 512, 2, 64, 128, 1, 256, bf, 2, x, NULL, dt, A, (float*)ws, (float*)y, C, (float*)D, (float*)init, NULL) == SSD_ERR_NULL);
    CHECK(ssd_run_passing(1, 512, 2, 64, 128, 256, bf, 2, NULL, dt, init, y, fin, NULL) == SSD_ERR_NULL);
    CHECK(ssd_run_passing(1, 512, 2, 64, 128, 256, bf, -5, ws, dt, init, y, fin, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_chunk_scan_runs(1, 512, 2, 64, 128, 1, 256, bf, 2, x, B, C, dt, A, ws, y, (float*)D, NULL, NULL, NULL) == SSD_ERR_NULL);
    CHECK(ssd_chunk_scan_runs(1, 512, 2, 64, 128, 1, 256, f32, 2, x, B, C, dt, A, ws, y, (float*)D, NULL, fin, NULL) == SSD_ERR_UNSUPPORTED);

    /* the block around the scan */
    CHECK(ssd_layer_in(0, L, H, P, N, G, 4, f32, x, dt, NULL, A, NULL, y, B, C, fin, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_layer_in(b, L, H, P, N, G, 4, f32, NULL, dt, NULL, A, NULL, y, B, C, fin, NULL) == SSD_ERR_NULL);
    CHECK(ssd_layer_out(0, SSD_DTYPE_BF16, x, B, y, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_layer_out(16, SSD_DTYPE_BF16, NULL, B, y, NULL) == SSD_ERR_NULL);
}

#endif

#ifdef CHECK_ORACLE
/* splitmix64: seeded uniform draws for the oracle inputs */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) {
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

/* bf16 bit pattern of a float (truncation: any bf16 value will do here) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void oracle_checks(int32_t kind, int32_t zoh) {
    const int64_t b = 2, L = 37, H = 4, P = 5, N = 6, G = 2;
    const size_t es = kind == 0 ? 4 : 2;
    const int64_t nx = b * L * H * P, nb = b * L * G * N, nd = b * L * H;
    unsigned char* x = malloc((size_t)nx * es);
    unsigned char* Bm = malloc((size_t)nb * es);
    unsigned char* Cm = malloc((size_t)nb * es);
    float* dt = malloc((size_t)nd * sizeof(float));
    float A[4], D[4];
    float* init = malloc((size_t)(b * H * P * N) * sizeof(float));
    for (int64_t i = 0; i < nx; ++i) {
        const float v = (float)(2.0 * uniform() - 1.0);
        if (kind == 0) memcpy(x + 4 * i, &v, 4);
        else { const uint16_t h = to_bf16(v); memcpy(x + 2 * i, &h, 2); }
    }
    for (int64_t i = 0; i < nb; ++i) {
        const float v = (float)(uniform() - 0.5), w = (float)(uniform() - 0.5);
        if (kind == 0) { memcpy(Bm + 4 * i, &v, 4); memcpy(Cm + 4 * i, &w, 4); }
        else { const uint16_t h = to_bf16(v), k = to_bf16(w); memcpy(Bm + 2 * i, &h, 2); memcpy(Cm + 2 * i, &k, 2); }
    }
    for (int64_t i = 0; i < nd; ++i) dt[i] = (float)(0.5 * uniform());
    for (int h = 0; h < H; ++h) { A[h] = (float)(-2.0 * uniform()); D[h] = (float)(uniform() - 0.5); }
    A[0] = 0.0f;   /* the A = 0 limit of the zero-order hold */
    for (int64_t i = 0; i < b * H * P * N; ++i) init[i] = (float)(0.1 * (uniform() - 0.5));

    int64_t bh[2 * 8];
    for (int64_t k = 0; k < b * H; ++k) { bh[2 * k] = k / H; bh[2 * k + 1] = k % H; }
    double* y_fwd = malloc((size_t)(b * H * L * P) * sizeof(double));
    double* f_fwd = malloc((size_t)(b * H * P * N) * sizeof(double));
    CHECK(oracle_ssd_forward_ex(b, L, H, P, N, G, kind, x, dt, A, Bm, Cm, D, init, bh, b * H, 0, L,
                                y_fwd, f_fwd, zoh) == 0);
    /* bad arguments are refused */
    CHECK(oracle_ssd_forward_ex(b, L, 3, P, N, G, kind, x, dt, A, Bm, Cm, D, init, bh, 1, 0, L, y_fwd, f_fwd, zoh) < 0);
    CHECK(oracle_ssd_forward_ex(b, L, H, P, N, G, kind, x, dt, A, Bm, Cm, D, init, bh, 1, 0, L + 1, y_fwd, f_fwd, zoh) < 0);

    /* the same tokens one step at a time */
    double* st = malloc((size_t)(b * H * P * N) * sizeof(double));
    for (int64_t i = 0; i < b * H * P * N; ++i) st[i] = (double)init[i];
    unsigned char* xt = malloc((size_t)(b * H * P) * es);
    unsigned char* bt = malloc((size_t)(b * G * N) * es);
    unsigned char* ct = malloc((size_t)(b * G * N) * es);
    float* dtt = malloc((size_t)(b * H) * sizeof(float));
    double* yt = malloc((size_t)(b * H * P) * sizeof(double));
    double worst = 0.0;
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t bb = 0; bb < b; ++bb) {
            memcpy(xt + (size_t)(bb * H * P) * es, x + (size_t)((bb * L + t) * H * P) * es, (size_t)(H * P) * es);
            memcpy(bt + (size_t)(bb * G * N) * es, Bm + (size_t)((bb * L + t) * G * N) * es, (size_t)(G * N) * es);
            memcpy(ct + (size_t)(bb * G * N) * es, Cm + (size_t)((bb * L + t) * G * N) * es, (size_t)(G * N) * es);
            memcpy(dtt + bb * H, dt + (bb * L + t) * H, (size_t)H * sizeof(float));
        }
        CHECK(oracle_ssm_step_ex(b, H, P, N, G, kind, st, xt, dtt, A, bt, ct, D, yt, zoh) == 0);
        for (int64_t k = 0; k < b * H; ++k)
            for (int64_t p = 0; p < P; ++p) {
                const double d = fabs(yt[k * P + p] - y_fwd[(k * L + t) * P + p]);
                if (d > worst) worst = d;
            }
    }
    for (int64_t i = 0; i < b * H * P * N; ++i) {
        const double d = fabs(st[i] - f_fwd[i]);
        if (d > worst) worst = d;
    }
    CHECK(worst <= 1e-12);
    free(x); free(Bm); free(Cm); free(dt); free(init); free(y_fwd); free(f_fwd);
    free(st); free(xt); free(bt); free(ct); free(dtt); free(yt);
}

#endif

int main(void) {
#ifdef CHECK_LIBRARY
    library_checks();
#endif
#ifdef CHECK_ORACLE
    for (int32_t kind = 0; kind < 2; ++kind)
        for (int32_t zoh = 0; zoh < 2; ++zoh) oracle_checks(kind, zoh);
#endif
    printf(fails ? "host_checks: %d failures\n" : "host_checks: ok\n", fails);
    return fails != 0;
}
