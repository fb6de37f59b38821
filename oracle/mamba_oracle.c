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

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* d SiLU(v) / dv = s + v s (1 - s), s = sigmoid(v) */
static double dsilu(double v) { const double s = sigmoid(v); return s * (1.0 + v * (1.0 - s)); }

/*
 * Reverse mode of oracle_prefill: the gradients of a loss L whose gradient with respect
 * to y is dy (and which does not depend on the final states), with respect to every input
 * and to the initial states.  Nothing here comes from the pages beyond the forward step
 * above; the gradients are that step differentiated by the chain rule, token by token in
 * reverse order within each sequence (no information crosses a cu_seqlens boundary in
 * either direction).  With g = SiLU(z), p = C.h' + D u (so y = p g), a_n = exp(delta A_n),
 * and lambda_t = dL/dh'_t (the adjoint of the state after token t):
 *   dp_t       = dy_t g_t,          dz_t = dy_t p_t SiLU'(z_t)
 *   lambda_t   = dp_t C_t + a_{t+1} * lambda_{t+1}            (lambda_L = 0)
 *   dC_t[n]   += dp_t h'_t[n]                                  (summed over channels)
 *   dB_t[n]   += lambda_t[n] delta_t u_t                       (summed over channels)
 *   du_t       = dp_t D + delta_t sum_n lambda_t[n] B_t[n]
 *   ddelta_t   = u_t sum_n lambda_t[n] B_t[n] + sum_n lambda_t[n] h'_{t-1}[n] a_t[n] A_n
 *   dA_n      += lambda_t[n] h'_{t-1}[n] a_t[n] delta_t,        dA_log = dA * A
 *   dD        += dp_t u_t
 *   ddt_t      = ddelta_t sigmoid(dt_t + dt_bias),  ddt_bias += ddt_t
 *   dxc_t      = du_t SiLU'(xc_t),  dconv_b += dxc_t,  dconv_w[k] += dxc_t X(t-K+1+k)
 *   dX(m)     += dxc_t conv_w[k] for m = t-K+1+k: dx for m >= 0, the initial conv
 *                state's entry K-1+m for m < 0
 *   dh_init    = a_0 * lambda_0
 * Layouts as oracle_prefill; conv_state and ssm_state are the initial states (read only).
 * Outputs: dx, dz, ddt [T,d]; dB, dC [T,N]; dA_log [d,N]; dD, ddt_bias, dconv_b [d];
 * dconv_w [d,K]; dconv_state [S,d,K-1]; dssm_state [S,d,N].  All are overwritten.
 * Returns 0, or -1 for invalid arguments.  Serial (the outputs dB, dC and the parameter
 * gradients are sums over sequences and channels).
 */
int oracle_prefill_backward(int64_t T, int32_t S, int32_t d, int32_t N, int32_t K,
                            const double* x, const double* z, const double* dt, const double* B, const double* C,
                            const double* A_log, const double* D, const double* dt_bias,
                            const double* conv_w, const double* conv_b, const int32_t* cu_seqlens,
                            const double* conv_state, const double* ssm_state, const double* dy,
                            double* dx, double* dz, double* ddt, double* dB, double* dC, double* dA_log,
                            double* dD, double* ddt_bias, double* dconv_w, double* dconv_b,
                            double* dconv_state, double* dssm_state)
{
    if (T < 0 || S < 0 || d < 0 || N < 1 || K < 1 || K > ORACLE_MAX_K) return -1;
    if (S == 0) return T == 0 ? 0 : -1;
    if (cu_seqlens[0] != 0 || (int64_t)cu_seqlens[S] != T) return -1;
    for (int32_t s = 0; s < S; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    const int64_t KS = K - 1;
    memset(dx, 0, sizeof(double) * (size_t)(T * d));
    memset(dz, 0, sizeof(double) * (size_t)(T * d));
    memset(ddt, 0, sizeof(double) * (size_t)(T * d));
    memset(dB, 0, sizeof(double) * (size_t)(T * N));
    memset(dC, 0, sizeof(double) * (size_t)(T * N));
    memset(dA_log, 0, sizeof(double) * (size_t)d * N);
    memset(dD, 0, sizeof(double) * (size_t)d);
    memset(ddt_bias, 0, sizeof(double) * (size_t)d);
    memset(dconv_b, 0, sizeof(double) * (size_t)d);
    memset(dconv_w, 0, sizeof(double) * (size_t)d * K);
    memset(dconv_state, 0, sizeof(double) * (size_t)S * d * KS);
    memset(dssm_state, 0, sizeof(double) * (size_t)S * d * N);
    for (int32_t s = 0; s < S; ++s) {
        const int64_t g0 = cu_seqlens[s], L = cu_seqlens[s + 1] - g0;
        if (L == 0) continue;
        /* per-token forward quantities of this sequence (one channel at a time) */
        double* X = (double*)malloc(sizeof(double) * (size_t)(L + KS));  /* X[KS + m] = X(m), m >= -KS */
        double* xc = (double*)malloc(sizeof(double) * (size_t)L);
        double* u = (double*)malloc(sizeof(double) * (size_t)L);
        double* v = (double*)malloc(sizeof(double) * (size_t)L);
        double* dl = (double*)malloc(sizeof(double) * (size_t)L);
        double* p = (double*)malloc(sizeof(double) * (size_t)L);
        double* H = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N)); /* H[(t+1)N + n] = h'_t, H[n] = h_init */
        double* lam = (double*)malloc(sizeof(double) * (size_t)N);
        double* dxc = (double*)malloc(sizeof(double) * (size_t)L);
        double* A = (double*)malloc(sizeof(double) * (size_t)N);
        double* dA = (double*)malloc(sizeof(double) * (size_t)N);
        for (int32_t c = 0; c < d; ++c) {
            const double* w = conv_w + (int64_t)c * K;
            for (int n = 0; n < N; ++n) A[n] = -exp(A_log[(int64_t)c * N + n]);
            for (int64_t m = 0; m < KS; ++m) X[m] = conv_state[((int64_t)s * d + c) * KS + m];
            for (int64_t t = 0; t < L; ++t) X[KS + t] = x[(g0 + t) * d + c];
            for (int n = 0; n < N; ++n) H[n] = ssm_state[((int64_t)s * d + c) * N + n];
            /* forward */
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (g0 + t) * d + c;
                double acc = conv_b[c];
                for (int k = 0; k < K; ++k) acc += X[t + k] * w[k];  /* X(t-K+1+k) */
                xc[t] = acc;
                u[t] = silu(acc);
                v[t] = dt[i] + dt_bias[c];
                dl[t] = softplus(v[t]);
                double yp = D[c] * u[t];
                for (int n = 0; n < N; ++n) {
                    const double hn = exp(dl[t] * A[n]) * H[t * N + n] + dl[t] * B[(g0 + t) * N + n] * u[t];
                    H[(t + 1) * N + n] = hn;
                    yp += C[(g0 + t) * N + n] * hn;
                }
                p[t] = yp;
            }
            /* reverse */
            for (int n = 0; n < N; ++n) { lam[n] = 0.0; dA[n] = 0.0; }
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t i = (g0 + t) * d + c;
                const double g = silu(z[i]);
                const double dp = dy[i] * g;
                dz[i] = dy[i] * p[t] * dsilu(z[i]);
                double s1 = 0.0, s2 = 0.0;
                for (int n = 0; n < N; ++n) {
                    const double anext = (t + 1 < L) ? exp(dl[t + 1] * A[n]) : 0.0;
                    lam[n] = dp * C[(g0 + t) * N + n] + anext * lam[n];
                    const double a = exp(dl[t] * A[n]);
                    const double hprev = H[t * N + n];
                    dC[(g0 + t) * N + n] += dp * H[(t + 1) * N + n];
                    dB[(g0 + t) * N + n] += lam[n] * dl[t] * u[t];
                    s1 += lam[n] * B[(g0 + t) * N + n];
                    s2 += lam[n] * hprev * a * A[n];
                    dA[n] += lam[n] * hprev * a * dl[t];
                }
                dD[c] += dp * u[t];
                const double du = dp * D[c] + dl[t] * s1;
                const double ddelta = u[t] * s1 + s2;
                const double dv = ddelta * sigmoid(v[t]);
                ddt[i] = dv;
                ddt_bias[c] += dv;
                dxc[t] = du * dsilu(xc[t]);
            }
            for (int n = 0; n < N; ++n) {
                dA_log[(int64_t)c * N + n] += dA[n] * A[n];
                dssm_state[((int64_t)s * d + c) * N + n] = exp(dl[0] * A[n]) * lam[n];
            }
            /* conv */
            for (int64_t t = 0; t < L; ++t) {
                dconv_b[c] += dxc[t];
                for (int k = 0; k < K; ++k) {
                    dconv_w[(int64_t)c * K + k] += dxc[t] * X[t + k];
                    const int64_t m = t - KS + k;  /* the input this tap reads */
                    if (m >= 0) dx[(g0 + m) * d + c] += dxc[t] * w[k];
                    else dconv_state[((int64_t)s * d + c) * KS + (KS + m)] += dxc[t] * w[k];
                }
            }
        }
        free(X); free(xc); free(u); free(v); free(dl); free(p); free(H); free(lam); free(dxc); free(A); free(dA);
    }
    return 0;
}
