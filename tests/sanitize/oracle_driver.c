/*
 * oracle_driver.c -- the C oracle (oracle/gdn_oracle.c) under AddressSanitizer
 * and UndefinedBehaviorSanitizer, on the CPU: prefills over packed sequences
 * (empty ones included) in fp64, fp32 and bf16 storage, a subset of state rows,
 * several threads, decode steps, and the argument checks.  Values are checked
 * against two closed forms of the recurrence (identity gates keep the state;
 * unit keys with alpha = beta = 1 recall v exactly).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_prefill_f64(const void* q, const void* k, const void* v, int qkv_dt, const void* g, const void* beta,
                       int gate_dt, const void* init_state, int state_dt, const int64_t* cu_seqlens, int32_t N,
                       int32_t H, int32_t dk, int32_t dv, double scale, int32_t qk_l2norm, double eps,
                       const int32_t* rows, int32_t n_rows, double* o, double* final_state, int32_t n_threads,
                       int32_t mutation);
int oracle_decode_f64(const void* q, const void* k, const void* v, int qkv_dt, const void* g, const void* beta,
                      int gate_dt, double* state, int32_t N, int32_t H, int32_t dk, int32_t dv, double scale,
                      int32_t qk_l2norm, double eps, double* o, int32_t n_threads);

static int fails = 0;
#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++fails;                                                           \
        }                                                                      \
    } while (0)

static double urand(uint64_t* s)
{
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((*s >> 11) * (1.0 / 9007199254740992.0)) * 2.0 - 1.0;
}

int main(void)
{
    uint64_t seed = 12345;
    const int32_t H = 2, dk = 8, dv = 6, N = 4;
    const int64_t cu[5] = {0, 9, 9, 30, 31};
    const int64_t T = 31;
    double *q = malloc(sizeof(double) * T * H * dk), *k = malloc(sizeof(double) * T * H * dk);
    double *v = malloc(sizeof(double) * T * H * dv), *g = malloc(sizeof(double) * T * H), *b = malloc(sizeof(double) * T * H);
    double *s0 = malloc(sizeof(double) * N * H * dv * dk), *o = malloc(sizeof(double) * T * H * dv);
    double *fs = malloc(sizeof(double) * N * H * dv * dk);
    for (int64_t i = 0; i < T * H * dk; ++i) { q[i] = urand(&seed); k[i] = urand(&seed); }
    for (int64_t i = 0; i < T * H * dv; ++i) v[i] = urand(&seed);
    for (int64_t i = 0; i < T * H; ++i) { g[i] = -fabs(urand(&seed)); b[i] = 0.5 + 0.4 * urand(&seed); }
    for (int64_t i = 0; i < N * H * dv * dk; ++i) s0[i] = urand(&seed);

    /* general case, several thread counts: identical results */
    CHECK(oracle_prefill_f64(q, k, v, 0, g, b, 0, s0, 0, cu, N, H, dk, dv, 0.3, 1, 1e-6, NULL, 0, o, fs, 1, 0) == 0);
    double* o2 = malloc(sizeof(double) * T * H * dv);
    double* fs2 = malloc(sizeof(double) * N * H * dv * dk);
    CHECK(oracle_prefill_f64(q, k, v, 0, g, b, 0, s0, 0, cu, N, H, dk, dv, 0.3, 1, 1e-6, NULL, 0, o2, fs2, 3, 0) == 0);
    CHECK(memcmp(o, o2, sizeof(double) * T * H * dv) == 0 && memcmp(fs, fs2, sizeof(double) * N * H * dv * dk) == 0);
    /* the empty sequence keeps its initial state */
    CHECK(memcmp(fs + 1 * H * dv * dk, s0 + 1 * H * dv * dk, sizeof(double) * H * dv * dk) == 0);
    /* a subset of rows equals those rows of the full run */
    const int32_t rows[2] = {1, 4};
    double* o3 = calloc((size_t)T * H * dv, sizeof(double));
    double* fs3 = calloc((size_t)N * H * dv * dk, sizeof(double));
    CHECK(oracle_prefill_f64(q, k, v, 0, g, b, 0, s0, 0, cu, N, H, dk, dv, 0.3, 1, 1e-6, rows, 2, o3, fs3, 2, 0) == 0);
    for (int64_t t = 0; t < T * H; ++t)
        for (int r = 0; r < 2; ++r) CHECK(o3[t * dv + rows[r]] == o[t * dv + rows[r]]);

    /* identity gates (g = 0, beta = 0): the state is unchanged */
    double* z = calloc((size_t)T * H, sizeof(double));
    CHECK(oracle_prefill_f64(q, k, v, 0, z, z, 0, s0, 0, cu, N, H, dk, dv, 1.0, 1, 1e-6, NULL, 0, o, fs, 2, 0) == 0);
    for (int64_t i = 0; i < N * H * dv * dk; ++i) CHECK(fs[i] == s0[i]);

    /* fp32 and bf16 storage of the same inputs */
    float* qf = malloc(sizeof(float) * T * H * dk);
    uint16_t* qb = malloc(sizeof(uint16_t) * T * H * dk);
    for (int64_t i = 0; i < T * H * dk; ++i) {
        qf[i] = (float)q[i];
        uint32_t u;
        memcpy(&u, &qf[i], 4);
        qb[i] = (uint16_t)(u >> 16);
    }
    float* gf = malloc(sizeof(float) * T * H);
    float* bf = malloc(sizeof(float) * T * H);
    for (int64_t i = 0; i < T * H; ++i) { gf[i] = (float)g[i]; bf[i] = (float)b[i]; }
    double* o4 = malloc(sizeof(double) * T * H * dk);           /* d_v = d_k here */
    double* fs4 = malloc(sizeof(double) * N * H * dk * dk);
    CHECK(oracle_prefill_f64(qf, qf, qf, 1, gf, bf, 1, NULL, 0, cu, N, H, dk, dk, 0.3, 1, 1e-6, NULL, 0, o4, fs4, 2, 0) == 0);
    CHECK(oracle_prefill_f64(qb, qb, qb, 2, gf, bf, 1, NULL, 0, cu, N, H, dk, dk, 0.3, 0, 0.0, NULL, 0, o4, fs4, 2, 0) == 0);
    free(o4);
    free(fs4);

    /* decode: alpha = beta = 1 and a unit key recall v exactly */
    {
        const int32_t Nd = 3, d = 8;
        double* st = calloc((size_t)Nd * H * d * d, sizeof(double));
        double *kk = calloc((size_t)Nd * H * d, sizeof(double)), *vv = malloc(sizeof(double) * Nd * H * d);
        double *ones = malloc(sizeof(double) * Nd * H), *zeros = calloc((size_t)Nd * H, sizeof(double));
        double* od = malloc(sizeof(double) * Nd * H * d);
        for (int i = 0; i < Nd * H; ++i) { kk[i * d + (i % d)] = 1.0; ones[i] = 1.0; }
        for (int i = 0; i < Nd * H * d; ++i) vv[i] = urand(&seed);
        CHECK(oracle_decode_f64(kk, kk, vv, 0, zeros, ones, 0, st, Nd, H, d, d, 1.0, 0, 0.0, od, 2) == 0);
        for (int i = 0; i < Nd * H; ++i)
            for (int r = 0; r < d; ++r) CHECK(od[i * d + r] == vv[i * d + r]);
        free(st); free(kk); free(vv); free(ones); free(zeros); free(od);
    }

    /* argument checks */
    const int64_t bad[3] = {0, 10, 5};
    CHECK(oracle_prefill_f64(q, k, v, 0, g, b, 0, NULL, 0, bad, 2, H, dk, dv, 1.0, 1, 1e-6, NULL, 0, o, NULL, 1, 0) == -1);
    const int32_t badrow[1] = {dv};
    CHECK(oracle_prefill_f64(q, k, v, 0, g, b, 0, NULL, 0, cu, N, H, dk, dv, 1.0, 1, 1e-6, badrow, 1, o, NULL, 1, 0) == -1);
    CHECK(oracle_prefill_f64(q, k, v, 0, g, b, 0, NULL, 0, cu, N, H, dk, dv, 1.0, 1, 1e-6, NULL, 0, o, NULL, 1, 99) == -1);

    free(q); free(k); free(v); free(g); free(b); free(s0); free(o); free(fs); free(o2); free(fs2); free(o3);
    free(fs3); free(z); free(qf); free(qb); free(gf); free(bf);
    printf("oracle driver: %d failed checks\n", fails);
    return fails == 0 ? 0 : 1;
}
