/*
 * Drives every entry point of the fp64 oracle (oracle/attention.c) on small
 * inputs held in exactly sized heap buffers, for a build with
 * -fsanitize=address,undefined: an access one element outside any buffer, a
 * use after free, a leak or undefined arithmetic ends the run with a report.
 * It also checks a few results the definition fixes (finite outputs on visible
 * rows, -inf LSE on empty rows, identical keys give the mean of the visible
 * values) and that bad arguments are refused.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                          int B, int H, int Nq, int Nk, int d, int causal, float scale,
                          int key_begin, int key_end, const int64_t *rows, int64_t nrows,
                          double *o, double *lse, int nthreads);
int oracle_attention_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                            int B, int H, int H_kv, int d, const int32_t *cu_q, const int32_t *cu_k,
                            int causal, float scale, const int64_t *rows, int64_t nrows,
                            double *o, double *lse, int nthreads);
int oracle_combine(const double *o_part, const double *lse_part, int S, int64_t R, int d,
                   double *o, double *lse);
int oracle_attention_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                         int dtype, int B, int H, int Nq, int Nk, int d, int causal, float scale,
                         const int64_t *q_rows, int64_t n_q, const int64_t *k_rows, int64_t n_k,
                         double *dq, double *dk, double *dv, int nthreads);

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
            ++failures;                                    \
        }                                                  \
    } while (0)

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {   /* xorshift32 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}

/* Random 16-bit patterns of moderate finite values: fp16 exponents 12..16
 * (0.125..2) or bf16 exponents 124..128, random sign and fraction. */
static uint16_t *rand_bits(size_t n, int dtype) {
    uint16_t *x = (uint16_t *)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        uint32_t r = next_u32();
        uint16_t sign = (uint16_t)((r & 1u) << 15);
        uint16_t e = (uint16_t)((r >> 1) % 5u);
        if (dtype == 0)
            x[i] = sign | (uint16_t)((12 + e) << 10) | (uint16_t)((r >> 8) & 0x3FF);
        else
            x[i] = sign | (uint16_t)((124 + e) << 7) | (uint16_t)((r >> 8) & 0x7F);
    }
    return x;
}

static double *dalloc(size_t n) { return (double *)malloc((n ? n : 1) * sizeof(double)); }

static void check_rows(const double *o, const double *lse, int64_t n, int d, const char *what) {
    for (int64_t r = 0; r < n; ++r) {
        if (isinf(lse[r])) {
            CHECK(lse[r] < 0, "%s: +inf LSE at row %lld", what, (long long)r);
            for (int t = 0; t < d; ++t) CHECK(o[r * d + t] == 0.0, "%s: empty row %lld has O != 0", what, (long long)r);
        } else {
            CHECK(isfinite(lse[r]), "%s: LSE not finite at row %lld", what, (long long)r);
            for (int t = 0; t < d; ++t) CHECK(isfinite(o[r * d + t]), "%s: O not finite at row %lld", what, (long long)r);
        }
    }
}

static void dense_cases(void) {
    const int shapes[][5] = {  /* B, H, Nq, Nk, d */
        {1, 1, 1, 1, 8}, {2, 3, 17, 33, 16}, {1, 2, 40, 9, 8}, {1, 1, 64, 64, 64}, {2, 1, 5, 130, 128},
    };
    for (size_t c = 0; c < sizeof(shapes) / sizeof(shapes[0]); ++c)
        for (int dtype = 0; dtype < 2; ++dtype)
            for (int causal = 0; causal < 2; ++causal) {
                const int B = shapes[c][0], H = shapes[c][1], Nq = shapes[c][2], Nk = shapes[c][3], d = shapes[c][4];
                const int64_t R = (int64_t)B * H * Nq;
                uint16_t *q = rand_bits((size_t)R * d, dtype);
                uint16_t *k = rand_bits((size_t)B * H * Nk * d, dtype);
                uint16_t *v = rand_bits((size_t)B * H * Nk * d, dtype);
                double *o = dalloc((size_t)R * d), *lse = dalloc((size_t)R);
                CHECK(oracle_attention_rows(q, k, v, dtype, B, H, Nq, Nk, d, causal, 0.3f, 0, Nk, NULL, R, o, lse,
                                            (int)(c % 3) + 1) == 0, "rows call");
                check_rows(o, lse, R, d, "dense");
                /* a key range and a subset of rows */
                int64_t rows[3] = {0, R - 1, R / 2};
                double *o2 = dalloc(3 * (size_t)d), *l2 = dalloc(3);
                CHECK(oracle_attention_rows(q, k, v, dtype, B, H, Nq, Nk, d, causal, -0.7f, Nk / 3, Nk - Nk / 4,
                                            rows, 3, o2, l2, 2) == 0, "rows subset call");
                check_rows(o2, l2, 3, d, "dense subset");
                /* split partials and their combine */
                const int S = 3, chunk = (Nk + S - 1) / S;
                double *op = dalloc((size_t)S * R * d), *lp = dalloc((size_t)S * R);
                for (int s = 0; s < S; ++s)
                    CHECK(oracle_attention_rows(q, k, v, dtype, B, H, Nq, Nk, d, causal, 0.3f, s * chunk,
                                                (s + 1) * chunk, NULL, R, op + (size_t)s * R * d, lp + (size_t)s * R,
                                                1) == 0, "split call");
                double *oc = dalloc((size_t)R * d), *lc = dalloc((size_t)R);
                CHECK(oracle_combine(op, lp, S, R, d, oc, lc) == 0, "combine call");
                for (int64_t i = 0; i < R * d; ++i) CHECK(fabs(oc[i] - o[i]) < 1e-12, "combine != unsplit O");
                /* backward over every row, then over sampled rows */
                uint16_t *g = rand_bits((size_t)R * d, dtype);
                const int64_t RK = (int64_t)B * H * Nk;
                double *dq = dalloc((size_t)R * d), *dk = dalloc((size_t)RK * d), *dv = dalloc((size_t)RK * d);
                CHECK(oracle_attention_bwd(q, k, v, g, dtype, B, H, Nq, Nk, d, causal, 0.3f, NULL, R, NULL, RK,
                                           dq, dk, dv, 3) == 0, "bwd call");
                for (int64_t i = 0; i < R * d; ++i) CHECK(isfinite(dq[i]), "dq not finite");
                for (int64_t i = 0; i < RK * d; ++i) CHECK(isfinite(dk[i]) && isfinite(dv[i]), "dk/dv not finite");
                int64_t krows[2] = {RK - 1, 0};
                double *dq2 = dalloc(3 * (size_t)d), *dk2 = dalloc(2 * (size_t)d), *dv2 = dalloc(2 * (size_t)d);
                CHECK(oracle_attention_bwd(q, k, v, g, dtype, B, H, Nq, Nk, d, causal, 0.3f, rows, 3, krows, 2,
                                           dq2, dk2, dv2, 2) == 0, "bwd rows call");
                for (int t = 0; t < d; ++t) {
                    CHECK(dq2[t] == dq[t], "bwd row subset dq");
                    CHECK(dk2[t] == dk[(RK - 1) * d + t] && dv2[d + t] == dv[t], "bwd row subset dk/dv");
                }
                free(q); free(k); free(v); free(o); free(lse); free(o2); free(l2); free(op); free(lp);
                free(oc); free(lc); free(g); free(dq); free(dk); free(dv); free(dq2); free(dk2); free(dv2);
            }
}

static void identical_keys(void) {
    /* every key equal: O_i is the mean of the visible values (causal: v_0..v_i) */
    const int Nq = 12, Nk = 12, d = 8;
    uint16_t *q = rand_bits((size_t)Nq * d, 0), *k = rand_bits((size_t)Nk * d, 0), *v = rand_bits((size_t)Nk * d, 0);
    for (int j = 1; j < Nk; ++j) memcpy(k + (size_t)j * d, k, (size_t)d * sizeof(uint16_t));
    double *o = dalloc((size_t)Nq * d), *lse = dalloc(Nq), *vd = dalloc((size_t)Nk * d);
    CHECK(oracle_attention_rows(q, k, v, 0, 1, 1, Nq, Nk, d, 1, 0.5f, 0, Nk, NULL, Nq, o, lse, 1) == 0, "call");
    /* decode the values with an all-ones query against one key: scale 0 gives the plain mean */
    double *om = dalloc((size_t)Nq * d), *lm = dalloc(Nq);
    CHECK(oracle_attention_rows(q, k, v, 0, 1, 1, Nq, Nk, d, 1, 0.0f, 0, Nk, NULL, Nq, om, lm, 1) == 0, "call");
    for (int i = 0; i < Nq; ++i) {
        for (int t = 0; t < d; ++t) CHECK(fabs(o[i * d + t] - om[i * d + t]) < 1e-12, "identical keys: O is the mean");
        CHECK(fabs(lm[i] - log((double)(i + 1))) < 1e-12, "scale 0: LSE = ln |V_i|");
    }
    free(q); free(k); free(v); free(o); free(lse); free(vd); free(om); free(lm);
}

static void varlen_cases(void) {
    const int B = 4, H = 4, H_kv = 2, d = 16;
    const int32_t cu_q[5] = {0, 7, 7, 40, 41};       /* an empty sequence and a one-row one */
    const int32_t cu_k[5] = {0, 9, 20, 20, 57};      /* one with no keys */
    for (int dtype = 0; dtype < 2; ++dtype)
        for (int causal = 0; causal < 2; ++causal) {
            const int64_t R = (int64_t)cu_q[B] * H;
            uint16_t *q = rand_bits((size_t)R * d, dtype);
            uint16_t *k = rand_bits((size_t)cu_k[B] * H_kv * d, dtype);
            uint16_t *v = rand_bits((size_t)cu_k[B] * H_kv * d, dtype);
            double *o = dalloc((size_t)R * d), *lse = dalloc((size_t)R);
            CHECK(oracle_attention_varlen(q, k, v, dtype, B, H, H_kv, d, cu_q, cu_k, causal, 0.25f, NULL, R, o, lse,
                                          3) == 0, "varlen call");
            check_rows(o, lse, R, d, "varlen");
            for (int h = 0; h < H; ++h) CHECK(isinf(lse[(7 + 10) * H + h]), "sequence without keys: LSE = -inf");
            free(q); free(k); free(v); free(o); free(lse);
        }
}

static void bad_arguments(void) {
    uint16_t *x = rand_bits(64, 0);
    double *o = dalloc(64), *l = dalloc(8);
    int64_t bad_row = 8;
    CHECK(oracle_attention_rows(x, x, x, 0, 1, 1, 8, 8, 8, 0, 1.f, 0, 8, &bad_row, 1, o, l, 1) == -1, "row out of range");
    CHECK(oracle_attention_rows(x, x, x, 2, 1, 1, 8, 8, 8, 0, 1.f, 0, 8, NULL, 8, o, l, 1) == -1, "bad dtype");
    CHECK(oracle_attention_rows(NULL, x, x, 0, 1, 1, 8, 8, 8, 0, 1.f, 0, 8, NULL, 8, o, l, 1) == -1, "null q");
    const int32_t cu_bad[3] = {0, 5, 3};
    CHECK(oracle_attention_varlen(x, x, x, 0, 2, 1, 1, 8, cu_bad, cu_bad, 0, 1.f, NULL, 3, o, l, 1) == -1,
          "decreasing offsets");
    CHECK(oracle_combine(o, l, 0, 1, 8, o, l) == -1, "no splits");
    free(x); free(o); free(l);
}

int main(void) {
    dense_cases();
    identical_keys();
    varlen_cases();
    bad_arguments();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run ok\n");
    return 0;
}
