/*
 * The oracle's C routines under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Every array is allocated at exactly its documented size, so that a read or write one
 * element past its end is reported.  The cases cover the paths through the routines: empty
 * sequences, sequences shorter than the conv window, a state wider than the on-stack buffer
 * (N > 256), the smallest and largest conv widths, T == 0, and the invalid arguments that
 * must be refused (-1) without touching any array.  Prefill, decode and the backward run on
 * each; the results are checked for finiteness and, for the prefill, against a token-by-token
 * chain of decode steps (the two routines are written separately).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_prefill(int64_t T, int32_t S, int32_t d, int32_t N, int32_t K, const double* x, const double* z,
                   const double* dt, const double* B, const double* C, const double* A_log, const double* D,
                   const double* dt_bias, const double* conv_w, const double* conv_b, const int32_t* cu_seqlens,
                   double* conv_state, double* ssm_state, double* y, int nthreads);
int oracle_decode(int32_t Bs, int32_t d, int32_t N, int32_t K, const double* x, const double* z, const double* dt,
                  const double* B, const double* C, const double* A_log, const double* D, const double* dt_bias,
                  const double* conv_w, const double* conv_b, double* conv_state, double* ssm_state, double* y,
                  int nthreads);
int oracle_prefill_backward(int64_t T, int32_t S, int32_t d, int32_t N, int32_t K, const double* x,
                            const double* z, const double* dt, const double* B, const double* C,
                            const double* A_log, const double* D, const double* dt_bias, const double* conv_w,
                            const double* conv_b, const int32_t* cu_seqlens, const double* conv_state,
                            const double* ssm_state, const double* dy, double* dx, double* dz, double* ddt,
                            double* dB, double* dC, double* dA_log, double* dD, double* ddt_bias, double* dconv_w,
                            double* dconv_b, double* dconv_state, double* dssm_state);

static int failures = 0;
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* xorshift64*, mapped to [-1, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* exactly n doubles (one byte for n == 0, so that the pointer is valid and unique) */
static double* arr(int64_t n) {
    double* p = (double*)malloc(n > 0 ? sizeof(double) * (size_t)n : 1);
    for (int64_t i = 0; i < n; ++i) p[i] = uniform();
    return p;
}

static int finite(const double* p, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static void check_case(const char* name, int S, const int32_t* lens, int d, int N, int K) {
    int64_t T = 0;
    for (int s = 0; s < S; ++s) T += lens[s];
    int32_t* cu = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
    cu[0] = 0;
    for (int s = 0; s < S; ++s) cu[s + 1] = cu[s] + lens[s];
    const int64_t KS = K - 1;
    double *x = arr(T * d), *z = arr(T * d), *dt = arr(T * d), *B = arr(T * N), *C = arr(T * N);
    double *A_log = arr((int64_t)d * N), *D = arr(d), *dtb = arr(d), *w = arr((int64_t)d * K), *b = arr(d);
    double *cs = arr((int64_t)S * d * KS), *ss = arr((int64_t)S * d * N), *y = arr(T * d);
    double *cs0 = arr((int64_t)S * d * KS), *ss0 = arr((int64_t)S * d * N);
    memcpy(cs0, cs, sizeof(double) * (size_t)(S * d * KS));
    memcpy(ss0, ss, sizeof(double) * (size_t)(S * d * N));
    int rc = oracle_prefill(T, S, d, N, K, x, z, dt, B, C, A_log, D, dtb, w, b, cu, cs, ss, y, 2);
    if (rc != 0 || !finite(y, T * d) || !finite(ss, (int64_t)S * d * N)) {
        printf("FAIL %s: prefill rc %d\n", name, rc);
        ++failures;
    }
    /* the same tokens through decode steps, one sequence and one token at a time */
    double *x1 = arr(d), *z1 = arr(d), *dt1 = arr(d), *B1 = arr(N), *C1 = arr(N), *y1 = arr(d);
    double *csr = arr(d * KS), *ssr = arr((int64_t)d * N);
    double worst = 0.0;
    for (int s = 0; s < S; ++s) {
        memcpy(csr, cs0 + (int64_t)s * d * KS, sizeof(double) * (size_t)(d * KS));
        memcpy(ssr, ss0 + (int64_t)s * d * N, sizeof(double) * (size_t)(d * N));
        for (int64_t g = cu[s]; g < cu[s + 1]; ++g) {
            memcpy(x1, x + g * d, sizeof(double) * (size_t)d);
            memcpy(z1, z + g * d, sizeof(double) * (size_t)d);
            memcpy(dt1, dt + g * d, sizeof(double) * (size_t)d);
            memcpy(B1, B + g * N, sizeof(double) * (size_t)N);
            memcpy(C1, C + g * N, sizeof(double) * (size_t)N);
            if (oracle_decode(1, d, N, K, x1, z1, dt1, B1, C1, A_log, D, dtb, w, b, csr, ssr, y1, 1) != 0) {
                printf("FAIL %s: decode refused\n", name);
                ++failures;
            }
            for (int c = 0; c < d; ++c) worst = fmax(worst, fabs(y1[c] - y[g * d + c]));
        }
        for (int64_t i = 0; i < (int64_t)d * N; ++i) worst = fmax(worst, fabs(ssr[i] - ss[(int64_t)s * d * N + i]));
        for (int64_t i = 0; i < d * KS; ++i) worst = fmax(worst, fabs(csr[i] - cs[(int64_t)s * d * KS + i]));
    }
    if (!(worst <= 1e-12)) {
        printf("FAIL %s: prefill and decode chain differ by %g\n", name, worst);
        ++failures;
    }
    /* backward from the initial states */
    double *dy = arr(T * d), *dx = arr(T * d), *dz = arr(T * d), *ddt = arr(T * d), *dB = arr(T * N), *dC = arr(T * N);
    double *dA = arr((int64_t)d * N), *dD = arr(d), *ddtb = arr(d), *dw = arr((int64_t)d * K), *db = arr(d);
    double *dcs = arr((int64_t)S * d * KS), *dss = arr((int64_t)S * d * N);
    rc = oracle_prefill_backward(T, S, d, N, K, x, z, dt, B, C, A_log, D, dtb, w, b, cu, cs0, ss0, dy, dx, dz, ddt,
                                 dB, dC, dA, dD, ddtb, dw, db, dcs, dss);
    if (rc != 0 || !finite(dx, T * d) || !finite(dA, (int64_t)d * N) || !finite(dss, (int64_t)S * d * N)) {
        printf("FAIL %s: backward rc %d\n", name, rc);
        ++failures;
    }
    double* all[] = {x, z, dt, B, C, A_log, D, dtb, w, b, cs, ss, y, cs0, ss0, x1, z1, dt1, B1, C1, y1, csr, ssr,
                     dy, dx, dz, ddt, dB, dC, dA, dD, ddtb, dw, db, dcs, dss};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
    free(cu);
    printf("ok %s (T=%lld S=%d d=%d N=%d K=%d)\n", name, (long long)T, S, d, N, K);
}

static void check_refusals(void) {
    double* a = arr(64);
    int32_t bad_cu[3] = {0, 5, 3};  /* decreasing */
    int32_t off_cu[2] = {1, 4};     /* does not start at 0 */
    int32_t ok_cu[2] = {0, 4};
    struct { int64_t T; int32_t S, d, N, K; const int32_t* cu; } cases[] = {
        {-1, 1, 2, 2, 4, ok_cu}, {4, -1, 2, 2, 4, ok_cu}, {4, 1, -2, 2, 4, ok_cu}, {4, 1, 2, 0, 4, ok_cu},
        {4, 1, 2, 2, 0, ok_cu}, {4, 1, 2, 2, 65, ok_cu}, {4, 0, 2, 2, 4, ok_cu}, {3, 2, 2, 2, 4, bad_cu},
        {4, 1, 2, 2, 4, off_cu}, {5, 1, 2, 2, 4, ok_cu}};
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) {
        const int rc = oracle_prefill(cases[i].T, cases[i].S, cases[i].d, cases[i].N, cases[i].K, a, a, a, a, a, a,
                                      a, a, a, a, cases[i].cu, a, a, a, 1);
        const int rb = oracle_prefill_backward(cases[i].T, cases[i].S, cases[i].d, cases[i].N, cases[i].K, a, a, a,
                                               a, a, a, a, a, a, a, cases[i].cu, a, a, a, a, a, a, a, a, a, a, a,
                                               a, a, a, a);
        if (rc != -1 || rb != -1) {
            printf("FAIL refusal case %zu: prefill %d, backward %d\n", i, rc, rb);
            ++failures;
        }
    }
    if (oracle_decode(-1, 2, 2, 4, a, a, a, a, a, a, a, a, a, a, a, a, a, 1) != -1 ||
        oracle_decode(1, 2, 2, 99, a, a, a, a, a, a, a, a, a, a, a, a, a, 1) != -1) {
        printf("FAIL decode refusals\n");
        ++failures;
    }
    /* nothing to do */
    int32_t zero_cu[1] = {0};
    if (oracle_prefill(0, 0, 2, 2, 4, a, a, a, a, a, a, a, a, a, a, zero_cu, a, a, a, 1) != 0) {
        printf("FAIL empty prefill\n");
        ++failures;
    }
    free(a);
    printf("ok refusals\n");
}

int main(void) {
    const int32_t mix[] = {0, 2, 7, 1, 0, 19};
    check_case("mixed lengths with empty and short sequences", 6, mix, 5, 3, 4);
    const int32_t one[] = {3};
    check_case("state wider than the stack buffer", 1, one, 2, 300, 2);
    const int32_t two[] = {4, 9};
    check_case("conv width 1", 2, two, 3, 4, 1);
    check_case("conv width 64", 2, two, 3, 2, 64);
    const int32_t none[] = {0, 0};
    check_case("no tokens", 2, none, 4, 16, 4);
    const int32_t big[] = {40, 33};
    check_case("N = 16, d = 17", 2, big, 17, 16, 4);
    check_refusals();
    if (failures) {
        printf("%d failures\n", failures);
        return 1;
    }
    printf("all ok\n");
    return 0;
}
