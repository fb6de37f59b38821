/*
 * mamba_oracle.c -- slow, plain fp64 CPU oracle of the selective-SSM mixer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library and must never serve as a
 * fallback for it.
 *
 * What it computes, and where each step comes from:
 *
 *  - The one-token mixer step is the one spelled out by the TensorRT Mamba
 *    tensor-parallel builder (NVIDIA TensorRT-Model-Connect,
 *    families/mamba/tp_builder.py, function _add_mamba_tp_layer):
 *      window   = [previous K-1 raw inputs, current x]    (slice + concat, newest last)
 *      u        = SiLU(sum_k window[k] * conv_w[c,k] + conv_b[c])
 *      delta    = log(exp(dt + dt_bias) + 1)              (softplus of the biased dt)
 *      Abar     = exp(delta * A)                          (A per channel and state index)
 *      h'       = Abar * h + (delta * B) * u
 *      y        = h' . C + D * u                          (readout uses the updated state)
 *      out      = y * SiLU(z)
 *    The builder keeps K columns of conv state and drops the oldest on entry;
 *    the state kept here is the K-1 newest raw inputs (oldest first), which is
 *    the same information.
 *  - A = -exp(A_log) (the usual Mamba log-parameterisation of the decay).
 *  - A prefill over a sequence is that step applied token after token; the
 *    "Scaling State-Space Models on Multiple GPUs with Tensor Parallelism" page
 *    (abstract; Fig. 2 component (1), the SSM cache) carries the final conv and
 *    SSM state from prefill into decode, so each sequence starts from its slot
 *    and leaves its final state there.
 *  - Packed variable-length input (PackMamba page, abstract): sequences are laid
 *    end to end, delimited by cu_seqlens, and no information passes between
 *    them; here each sequence is simply run on its own, from its own slot.
 *
 * Everything is evaluated in double precision, one token at a time, with no
 * chunking, reordering or parallel prefix.  Softplus is evaluated as
 * max(v,0) + log1p(exp(-|v|)), which equals log(1 + exp(v)) exactly and does
 * not lose digits for v << 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_K 64

static double silu(double v) { return v / (1.0 + exp(-v)); }

static double softplus(double v) { return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v))); }

/* One mixer step for one channel.  win[0..K-2] holds the previous K-1 raw
 * inputs (oldest first) and is shifted in place to end with x.  h[0..N-1] is
 * the SSM state of the channel, updated in place.  Returns the gated output. */
static double mixer_step(int N, int K, double x, double z, double dt, const double* Bt, const double* Ct,
                         const double* A, double Dc, double dt_bias_c, const double* w, double b,
                         double* win, double* h)
{
    double window[ORACLE_MAX_K];
    for (int k = 0; k < K - 1; ++k) window[k] = win[k];
    window[K - 1] = x;
    double xc = b;
    for (int k = 0; k < K; ++k) xc += window[k] * w[k];
    for (int k = 0; k < K - 1; ++k) win[k] = window[k + 1];
    double u = silu(xc);
    double delta = softplus(dt + dt_bias_c);
    double yv = 0.0;
    for (int n = 0; n < N; ++n) {
        double abar = exp(delta * A[n]);
        h[n] = abar * h[n] + (delta * Bt[n]) * u;
        yv += h[n] * Ct[n];
    }
    yv += Dc * u;
    return yv * silu(z);
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int oracle_threads(int nthreads) { return set_threads(nthreads); }

/*
 * Prefill over S packed sequences.  Layouts (row-major, last index fastest):
 *   x, z, dt, y     [T, d]        B, C          [T, N]
 *   A_log           [d, N]        D, dt_bias, conv_b  [d]     conv_w [d, K]
 *   cu_seqlens      [S+1]  int32, cu[0] = 0, non-decreasing, cu[S] = T
 *   conv_state      [S, d, K-1]   in: initial raw inputs; out: final (in place)
 *   ssm_state       [S, d, N]     in: initial state;      out: final (in place)
 * Returns 0, or -1 for an invalid cu_seqlens / dims (nothing written then).
 */
int oracle_prefill(int64_t T, int32_t S, int32_t d, int32_t N, int32_t K,
                   const double* x, const double* z, const double* dt, const double* B, const double* C,
                   const double* A_log, const double* D, const double* dt_bias,
                   const double* conv_w, const double* conv_b, const int32_t* cu_seqlens,
                   double* conv_state, double* ssm_state, double* y, int nthreads)
{
    if (T < 0 || S < 0 || d < 0 || N < 1 || K < 1 || K > ORACLE_MAX_K) return -1;
    if (S == 0) return T == 0 ? 0 : -1;
    if (cu_seqlens[0] != 0 || (int64_t)cu_seqlens[S] != T) return -1;
    for (int32_t s = 0; s < S; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    set_threads(nthreads);
    const int64_t KS = K - 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int32_t s = 0; s < S; ++s) {
        for (int32_t c = 0; c < d; ++c) {
            const int64_t g0 = cu_seqlens[s], g1 = cu_seqlens[s + 1];
            if (g1 == g0) continue; /* empty sequence: slot untouched */
            double A[256];
            double* h = ssm_state + ((int64_t)s * d + c) * N;
            double* win = conv_state + ((int64_t)s * d + c) * KS;
            double* Ah = N <= 256 ? A : (double*)malloc(sizeof(double) * (size_t)N);
            for (int n = 0; n < N; ++n) Ah[n] = -exp(A_log[(int64_t)c * N + n]);
            for (int64_t g = g0; g < g1; ++g) {
                const int64_t i = g * d + c;
                y[i] = mixer_step(N, K, x[i], z[i], dt[i], B + g * N, C + g * N, Ah, D[c], dt_bias[c],
                                  conv_w + (int64_t)c * K, conv_b[c], win, h);
            }
            if (Ah != A) free(Ah);
        }
    }
    return 0;
}

/*
 * One decode step for Bs independent rows (row r uses slot r).  Layouts:
 *   x, z, dt, y [Bs, d]   B, C [Bs, N]   conv_state [Bs, d, K-1]   ssm_state [Bs, d, N]
 * The states are updated in place.  This is a routine of its own (not a call
 * of the prefill) so that "decode steps equal a prefill scan" is a real check.
 */
int oracle_decode(int32_t Bs, int32_t d, int32_t N, int32_t K,
                  const double* x, const double* z, const double* dt, const double* B, const double* C,
                  const double* A_log, const double* D, const double* dt_bias,
                  const double* conv_w, const double* conv_b,
                  double* conv_state, double* ssm_state, double* y, int nthreads)
{
    if (Bs < 0 || d < 0 || N < 1 || K < 1 || K > ORACLE_MAX_K) return -1;
    set_threads(nthreads);
    const int64_t KS = K - 1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t r = 0; r < Bs; ++r) {
        for (int32_t c = 0; c < d; ++c) {
            const int64_t i = (int64_t)r * d + c;
            double* h = ssm_state + i * N;
            double* win = conv_state + i * KS;
            /* conv window: the stored K-1 inputs, then this token's x */
            double window[ORACLE_MAX_K];
            for (int k = 0; k < K - 1; ++k) window[k] = win[k];
            window[K - 1] = x[i];
            double xc = conv_b[c];
            for (int k = 0; k < K; ++k) xc += window[k] * conv_w[(int64_t)c * K + k];
            /* drop the oldest entry, keep the newest K-1 */
            for (int k = 0; k < K - 1; ++k) win[k] = window[k + 1];
            const double u = silu(xc);
            const double delta = softplus(dt[i] + dt_bias[c]);
            double yv = 0.0;
            for (int n = 0; n < N; ++n) {
                const double a = -exp(A_log[(int64_t)c * N + n]);
                h[n] = exp(delta * a) * h[n] + (delta * B[(int64_t)r * N + n]) * u;
                yv += h[n] * C[(int64_t)r * N + n];
            }
            yv += D[c] * u;
            y[i] = yv * silu(z[i]);
        }
    }
    return 0;
}
