/*
 * Plain fp64 CPU oracle for the Hyena operator forward hot path and its backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code with the HIP library.
 *
 * What it computes (sources are the pages' own sections):
 *   - HyenaDNA walkthrough, section 2.1 (HyenaOperator code): the short filter is
 *     a depthwise width-3 convolution over every channel, padded by two and cut
 *     to the first L samples; its output splits into gates x_0..x_{N-1} and the
 *     value v (the last group of D channels); then for o = 0..N-2 the value is
 *     gated by x_{N-1-o} (the gates x_{N-1}..x_1 taken last to first) and passed
 *     through the long filter k[o] with bias[o]; finally y = v * x_0.
 *   - HyenaDNA walkthrough, section 2.2 (HyenaFilter code): the long filter step
 *     is an FFT convolution of the value with the filter and a bias, which the
 *     page equates with a per-channel Conv1d: a per-channel long convolution plus
 *     a bias term.
 *   - HyenaND summary, methodology (its boundary-handling item): the non-circular
 *     convolution is obtained by zero-padding to twice the length.
 * Readings taken where the pages are silent: the convolution is causal with zero
 * initial state, conv(v,h)[t] = sum_{s<=t} h[s] v[t-s]; the bias is a skip term
 * bias[o,d] * v applied to the gated input of the same step; the short-conv bias
 * is zero; dropout is the identity.
 *
 * Parity pins (closed forms, brute force, library special cases, invariants) live
 * in the test suite; every function below is checked against something other
 * than itself there.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PI 3.14159265358979323846264338327950288

/* Short depthwise convolution of one channel row: PyTorch Conv1d is a
 * cross-correlation, so with padding 2 the output at t is
 *   w[0]*u[t-2] + w[1]*u[t-1] + w[2]*u[t],   u[tau] = 0 for tau < 0,
 * and the first L outputs are kept (HyenaDNA walkthrough, section 2.1). */
void oracle_short_conv_row(const float* u, const float* w3, int64_t L, double* out) {
    for (int64_t t = 0; t < L; ++t) {
        double s = 0.0;
        for (int j = 0; j < 3; ++j) {
            int64_t tau = t - 2 + j;
            if (tau >= 0) s += (double)w3[j] * (double)u[tau];
        }
        out[t] = s;
    }
}

/* The same for a row given in fp64 (an intermediate the oracle computed itself). */
void oracle_short_conv_row64(const double* u, const float* w3, int64_t L, double* out) {
    for (int64_t t = 0; t < L; ++t) {
        double s = 0.0;
        for (int j = 0; j < 3; ++j) {
            int64_t tau = t - 2 + j;
            if (tau >= 0) s += (double)w3[j] * u[tau];
        }
        out[t] = s;
    }
}

/* Causal linear convolution by its definition: out[t] = sum_{s=0..t} h[s] v[t-s]. */
void oracle_causal_conv_direct(const double* v, const double* h, int64_t L, double* out) {
    for (int64_t t = 0; t < L; ++t) {
        double s = 0.0;
        for (int64_t k = 0; k <= t; ++k) s += h[k] * v[t - k];
        out[t] = s;
    }
}

/* Twiddle table for a length-n transform: tw[k] = exp(sign * 2 pi i k / n), k < n/2,
 * each value evaluated directly from cos/sin (no recurrence). */
static void make_twiddles(int64_t n, int sign, double* twr, double* twi) {
    for (int64_t k = 0; k < n / 2; ++k) {
        double ang = (double)sign * 2.0 * ORACLE_PI * (double)k / (double)n;
        twr[k] = cos(ang);
        twi[k] = sin(ang);
    }
}

/* Iterative radix-2 decimation-in-time FFT, in place, n a power of two.
 * sign = -1: X[k] = sum_t x[t] exp(-2 pi i k t / n)   (forward, unscaled)
 * sign = +1: x[t] = sum_k X[k] exp(+2 pi i k t / n)   (inverse, unscaled)
 * twr/twi must hold make_twiddles(n, sign). */
static void fft_radix2(double* re, double* im, int64_t n, const double* twr, const double* twi) {
    /* bit-reversal permutation */
    for (int64_t i = 1, j = 0; i < n; ++i) {
        int64_t bit = n >> 1;
        for (; j & bit; bit >>= 1) j ^= bit;
        j ^= bit;
        if (i < j) {
            double tr = re[i]; re[i] = re[j]; re[j] = tr;
            double ti = im[i]; im[i] = im[j]; im[j] = ti;
        }
    }
    /* butterflies: combine pairs of half-length transforms */
    for (int64_t len = 2; len <= n; len <<= 1) {
        int64_t half = len >> 1, step = n / len;
        for (int64_t base = 0; base < n; base += len) {
            for (int64_t k = 0; k < half; ++k) {
                double wr = twr[k * step], wi = twi[k * step];
                int64_t a = base + k, b = a + half;
                double xr = re[b] * wr - im[b] * wi;
                double xi = re[b] * wi + im[b] * wr;
                re[b] = re[a] - xr; im[b] = im[a] - xi;
                re[a] += xr;        im[a] += xi;
            }
        }
    }
}

/* Public single-transform entry (builds its own twiddles). Returns 0, or -1 if n is
 * not a power of two. */
int oracle_fft(double* re, double* im, int64_t n, int sign) {
    if (n < 1 || (n & (n - 1))) return -1;
    if (n == 1) return 0;
    double* twr = (double*)malloc(sizeof(double) * (size_t)(n / 2));
    double* twi = (double*)malloc(sizeof(double) * (size_t)(n / 2));
    make_twiddles(n, sign, twr, twi);
    fft_radix2(re, im, n, twr, twi);
    free(twr); free(twi);
    return 0;
}

static int64_t pow2_at_least(int64_t x) {
    int64_t n = 1;
    while (n < x) n <<= 1;
    return n;
}

/* Causal convolution through the FFT: zero-pad v and h to n >= 2L (a power of two),
 * multiply the spectra, invert, divide by n, keep the first L real samples.
 * Any n >= 2L-1 avoids wrap-around; this uses n = 2L for power-of-two L.
 * Scratch: 4*n doubles. Tables: twiddles of length n for both signs. */
static void conv_fft_with(const double* v, const double* h, int64_t L, int64_t n,
                          const double* fr, const double* fi, const double* ir, const double* ii,
                          double* scratch, double* out) {
    double *ar = scratch, *ai = scratch + n, *br = scratch + 2 * n, *bi = scratch + 3 * n;
    for (int64_t t = 0; t < n; ++t) {
        ar[t] = t < L ? v[t] : 0.0; ai[t] = 0.0;
        br[t] = t < L ? h[t] : 0.0; bi[t] = 0.0;
    }
    fft_radix2(ar, ai, n, fr, fi);
    fft_radix2(br, bi, n, fr, fi);
    for (int64_t k = 0; k < n; ++k) {
        double cr = ar[k] * br[k] - ai[k] * bi[k];
        double ci = ar[k] * bi[k] + ai[k] * br[k];
        ar[k] = cr; ai[k] = ci;
    }
    fft_radix2(ar, ai, n, ir, ii);
    for (int64_t t = 0; t < L; ++t) out[t] = ar[t] / (double)n;
}

void oracle_causal_conv_fft(const double* v, const double* h, int64_t L, double* out) {
    int64_t n = pow2_at_least(2 * L);
    double* tab = (double*)malloc(sizeof(double) * (size_t)(2 * n));
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(4 * n));
    make_twiddles(n, -1, tab, tab + n / 2);
    make_twiddles(n, +1, tab + n, tab + n + n / 2);
    conv_fft_with(v, h, L, n, tab, tab + n / 2, tab + n, tab + n + n / 2, scratch, out);
    free(tab); free(scratch);
}

/*
 * The forward hot path for a set of (b, d) rows.
 *   u     [B][(N+1)D][L]  fp32 values (bf16 inputs already widened exactly), or NULL
 *         when u64 (the same tensor in fp64) is given instead
 *   w     [(N+1)D][3]     short conv taps in PyTorch Conv1d order
 *   h     [N-1][D][L]     long filters
 *   bias  [N-1][D]
 *   rows  flat indices b*D + d to compute, or NULL for all B*D rows
 *   y     [nrows][L] in the order of `rows` (or [B][D][L] when rows == NULL)
 *   mode  0 = direct O(L^2) convolution, 1 = fp64 FFT convolution
 * Returns 0 on success, -1 on invalid arguments.
 */
int oracle_hyena_forward(int64_t B, int64_t D, int64_t L, int N,
                         const float* u, const double* u64, const float* w, const float* h, const float* bias,
                         const int64_t* rows, int64_t nrows, double* y, int mode, int nthreads) {
    if (B < 1 || D < 1 || L < 1 || N < 2 || (!u && !u64) || !w || !h || !bias || !y) return -1;
    if (mode != 0 && mode != 1) return -1;
    const int64_t C = (int64_t)(N + 1) * D;
    const int64_t total = rows ? nrows : B * D;
    if (rows) {
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= B * D) return -1;
    }
    const int64_t n = pow2_at_least(2 * L);
    double* tab = NULL;
    if (mode == 1) {
        tab = (double*)malloc(sizeof(double) * (size_t)(2 * n));
        make_twiddles(n, -1, tab, tab + n / 2);
        make_twiddles(n, +1, tab + n, tab + n + n / 2);
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        /* per-thread buffers: N gates + value + filter + conv result + FFT scratch */
        double* buf = (double*)malloc(sizeof(double) * (size_t)((N + 4) * L + (mode == 1 ? 4 * n : 0)));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        } else {
            double* xs = buf;                    /* x_0 .. x_{N-1}, each L */
            double* v = buf + (int64_t)N * L;    /* value branch */
            double* hk = v + L;                  /* current long filter, fp64 */
            double* c = hk + L;                  /* convolution result */
            double* scratch = c + L;
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < total; ++r) {
                const int64_t row = rows ? rows[r] : r;
                const int64_t b = row / D, d = row % D;
                /* short conv + split: channel i*D + d is x_i (i < N), channel N*D + d is v */
                for (int i = 0; i <= N; ++i) {
                    const int64_t ch = (int64_t)i * D + d;
                    double* dst = (i < N) ? xs + (int64_t)i * L : v;
                    if (u64) oracle_short_conv_row64(u64 + (b * C + ch) * L, w + ch * 3, L, dst);
                    else oracle_short_conv_row(u + (b * C + ch) * L, w + ch * 3, L, dst);
                }
                /* the recurrence: step o pairs gate x_{N-1-o} with k[o], bias[o] */
                for (int o = 0; o <= N - 2; ++o) {
                    const double* g = xs + (int64_t)(N - 1 - o) * L;
                    for (int64_t t = 0; t < L; ++t) v[t] *= g[t];
                    const float* hrow = h + ((int64_t)o * D + d) * L;
                    for (int64_t t = 0; t < L; ++t) hk[t] = (double)hrow[t];
                    if (mode == 0)
                        oracle_causal_conv_direct(v, hk, L, c);
                    else
                        conv_fft_with(v, hk, L, n, tab, tab + n / 2, tab + n, tab + n + n / 2, scratch, c);
                    const double bo = (double)bias[(int64_t)o * D + d];
                    for (int64_t t = 0; t < L; ++t) v[t] = c[t] + bo * v[t];
                }
                /* final gate */
                double* out = y + r * L;
                for (int64_t t = 0; t < L; ++t) out[t] = v[t] * xs[t];
            }
            free(buf);
        }
    }
    free(tab);
    return failed ? -1 : 0;
}

/*
 * Backward of the hot path (gradients of a scalar loss with upstream gradient dy
 * with respect to every input), by the chain rule on the same definitions.
 *
 * The adjoint of the causal convolution v -> conv(v, k) is the correlation
 *   corr(a, k)[t] = sum_{s=t}^{L-1} k[s-t] a[s],
 * and the gradient of conv(v, k) with respect to the kernel k, given the
 * upstream a, is corr(a, v) (same formula with the roles of k and v swapped).
 * With g_o = v_o * x_{N-1-o} and v_{o+1} = conv(g_o, h_o) + bias_o * g_o:
 *   dv_{N-1} = dy * x_0,                 dx_0 = dy * v_{N-1}
 *   for o = N-2 .. 0, with a = dv_{o+1}:
 *     dh_o    += corr(a, g_o)            dbias_o += sum_t a[t] g_o[t]
 *     dg_o     = corr(a, h_o) + bias_o * a
 *     dx_{N-1-o} = dg_o * v_o,           dv_o = dg_o * x_{N-1-o}
 * and through the short convolution uc = w0 u[t-2] + w1 u[t-1] + w2 u[t]:
 *   du[t] = w2 duc[t] + w1 duc[t+1] + w0 duc[t+2]   (samples past L-1 are 0)
 *   dw[j] += sum_t duc[t] u[t-2+j]                  (samples before 0 are 0)
 * Sums over the batch are taken for dh, dbias and dw.
 */

/* corr(a, k) by its definition, O(L^2). */
void oracle_causal_corr_direct(const double* a, const double* k, int64_t L, double* out) {
    for (int64_t t = 0; t < L; ++t) {
        double s = 0.0;
        for (int64_t q = t; q < L; ++q) s += k[q - t] * a[q];
        out[t] = s;
    }
}

/* corr(a, k) through the FFT on n >= 2L zero-padded points:
 * IFFT(FFT(a) * conj(FFT(k))) / n, first L samples (no wrap-around because the
 * negative lags land in the zero padding). Scratch: 4*n doubles. */
static void corr_fft_with(const double* a, const double* k, int64_t L, int64_t n,
                          const double* fr, const double* fi, const double* ir, const double* ii,
                          double* scratch, double* out) {
    double *ar = scratch, *ai = scratch + n, *br = scratch + 2 * n, *bi = scratch + 3 * n;
    for (int64_t t = 0; t < n; ++t) {
        ar[t] = t < L ? a[t] : 0.0; ai[t] = 0.0;
        br[t] = t < L ? k[t] : 0.0; bi[t] = 0.0;
    }
    fft_radix2(ar, ai, n, fr, fi);
    fft_radix2(br, bi, n, fr, fi);
    for (int64_t q = 0; q < n; ++q) {
        /* a * conj(b) */
        double cr = ar[q] * br[q] + ai[q] * bi[q];
        double ci = ai[q] * br[q] - ar[q] * bi[q];
        ar[q] = cr; ai[q] = ci;
    }
    fft_radix2(ar, ai, n, ir, ii);
    for (int64_t t = 0; t < L; ++t) out[t] = ar[t] / (double)n;
}

void oracle_causal_corr_fft(const double* a, const double* k, int64_t L, double* out) {
    int64_t n = pow2_at_least(2 * L);
    double* tab = (double*)malloc(sizeof(double) * (size_t)(2 * n));
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(4 * n));
    make_twiddles(n, -1, tab, tab + n / 2);
    make_twiddles(n, +1, tab + n, tab + n + n / 2);
    corr_fft_with(a, k, L, n, tab, tab + n / 2, tab + n, tab + n + n / 2, scratch, out);
    free(tab); free(scratch);
}

/*
 * Gradients of the hot path.
 *   inputs  u [B][(N+1)D][L], w [(N+1)D][3], h [N-1][D][L], bias [N-1][D] as in the
 *           forward, dy [B][D][L] (all fp32 values, widened exactly)
 *   outputs du [B][(N+1)D][L], dw [(N+1)D][3], dh [N-1][D][L], dbias [N-1][D] (fp64)
 *   mode    0 = direct O(L^2) convolutions and correlations, 1 = fp64 FFT
 * Channels d are independent (every output row belongs to one d), so the work is
 * split over d. Returns 0 on success, -1 on invalid arguments or allocation failure.
 */
int oracle_hyena_backward(int64_t B, int64_t D, int64_t L, int N,
                          const float* u, const float* w, const float* h, const float* bias,
                          const float* dy, double* du, double* dw, double* dh, double* dbias,
                          int mode, int nthreads) {
    if (B < 1 || D < 1 || L < 1 || N < 2 || !u || !w || !h || !bias || !dy) return -1;
    if (!du || !dw || !dh || !dbias) return -1;
    if (mode != 0 && mode != 1) return -1;
    const int64_t C = (int64_t)(N + 1) * D;
    const int64_t n = pow2_at_least(2 * L);
    double* tab = NULL;
    if (mode == 1) {
        tab = (double*)malloc(sizeof(double) * (size_t)(2 * n));
        make_twiddles(n, -1, tab, tab + n / 2);
        make_twiddles(n, +1, tab + n, tab + n + n / 2);
    }
    const double *fr = tab, *fi = tab ? tab + n / 2 : NULL, *ir = tab ? tab + n : NULL,
                 *ii = tab ? tab + n + n / 2 : NULL;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        /* x_0..x_{N-1}, v_0..v_{N-1}, g_0..g_{N-2}, duc_0..duc_N, filter, a, c, FFT scratch */
        const int64_t nbuf = (int64_t)(N + N + (N - 1) + (N + 1) + 3) * L + (mode == 1 ? 4 * n : 0);
        double* buf = (double*)malloc(sizeof(double) * (size_t)nbuf);
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        } else {
            double* xs = buf;
            double* vs = xs + (int64_t)N * L;
            double* gs = vs + (int64_t)N * L;
            double* duc = gs + (int64_t)(N - 1) * L;
            double* hk = duc + (int64_t)(N + 1) * L;
            double* a = hk + L;
            double* c = a + L;
            double* scratch = c + L;
#pragma omp for schedule(dynamic, 1)
            for (int64_t d = 0; d < D; ++d) {
                for (int i = 0; i <= N; ++i)
                    for (int j = 0; j < 3; ++j) dw[((int64_t)i * D + d) * 3 + j] = 0.0;
                for (int o = 0; o <= N - 2; ++o) {
                    dbias[(int64_t)o * D + d] = 0.0;
                    for (int64_t t = 0; t < L; ++t) dh[((int64_t)o * D + d) * L + t] = 0.0;
                }
                for (int64_t b = 0; b < B; ++b) {
                    /* forward, keeping every intermediate */
                    for (int i = 0; i <= N; ++i) {
                        const int64_t ch = (int64_t)i * D + d;
                        double* dst = (i < N) ? xs + (int64_t)i * L : vs;
                        oracle_short_conv_row(u + (b * C + ch) * L, w + ch * 3, L, dst);
                    }
                    for (int o = 0; o <= N - 2; ++o) {
                        const double* x = xs + (int64_t)(N - 1 - o) * L;
                        const double* vo = vs + (int64_t)o * L;
                        double* g = gs + (int64_t)o * L;
                        for (int64_t t = 0; t < L; ++t) g[t] = vo[t] * x[t];
                        const float* hrow = h + ((int64_t)o * D + d) * L;
                        for (int64_t t = 0; t < L; ++t) hk[t] = (double)hrow[t];
                        if (mode == 0) oracle_causal_conv_direct(g, hk, L, c);
                        else conv_fft_with(g, hk, L, n, fr, fi, ir, ii, scratch, c);
                        const double bo = (double)bias[(int64_t)o * D + d];
                        double* vn = vs + (int64_t)(o + 1) * L;
                        for (int64_t t = 0; t < L; ++t) vn[t] = c[t] + bo * g[t];
                    }
                    /* final gate y = v_{N-1} * x_0 */
                    const float* dyr = dy + (b * D + d) * L;
                    const double* vl = vs + (int64_t)(N - 1) * L;
                    for (int64_t t = 0; t < L; ++t) {
                        a[t] = (double)dyr[t] * xs[t];
                        duc[t] = (double)dyr[t] * vl[t];
                    }
                    /* the recurrence, last step first; a holds dv_{o+1} */
                    for (int o = N - 2; o >= 0; --o) {
                        const double* g = gs + (int64_t)o * L;
                        const double* x = xs + (int64_t)(N - 1 - o) * L;
                        const double* vo = vs + (int64_t)o * L;
                        double sb = 0.0;
                        for (int64_t t = 0; t < L; ++t) sb += a[t] * g[t];
                        dbias[(int64_t)o * D + d] += sb;
                        if (mode == 0) oracle_causal_corr_direct(a, g, L, c);
                        else corr_fft_with(a, g, L, n, fr, fi, ir, ii, scratch, c);
                        double* dho = dh + ((int64_t)o * D + d) * L;
                        for (int64_t t = 0; t < L; ++t) dho[t] += c[t];
                        const float* hrow = h + ((int64_t)o * D + d) * L;
                        for (int64_t t = 0; t < L; ++t) hk[t] = (double)hrow[t];
                        if (mode == 0) oracle_causal_corr_direct(a, hk, L, c);
                        else corr_fft_with(a, hk, L, n, fr, fi, ir, ii, scratch, c);
                        const double bo = (double)bias[(int64_t)o * D + d];
                        double* dx = duc + (int64_t)(N - 1 - o) * L;
                        for (int64_t t = 0; t < L; ++t) {
                            const double dg = c[t] + bo * a[t];
                            dx[t] = dg * vo[t];
                            a[t] = dg * x[t];
                        }
                    }
                    double* dv0 = duc + (int64_t)N * L;
                    for (int64_t t = 0; t < L; ++t) dv0[t] = a[t];
                    /* through the short convolution of every channel */
                    for (int i = 0; i <= N; ++i) {
                        const int64_t ch = (int64_t)i * D + d;
                        const double* dc = duc + (int64_t)i * L;
                        const float* ur = u + (b * C + ch) * L;
                        const float* w3 = w + ch * 3;
                        double* dur = du + (b * C + ch) * L;
                        for (int64_t t = 0; t < L; ++t) {
                            double s = 0.0;
                            for (int j = 0; j < 3; ++j) {
                                const int64_t q = t + 2 - j;
                                if (q < L) s += (double)w3[j] * dc[q];
                            }
                            dur[t] = s;
                        }
                        for (int j = 0; j < 3; ++j) {
                            double s = 0.0;
                            for (int64_t t = 0; t < L; ++t) {
                                const int64_t q = t - 2 + j;
                                if (q >= 0) s += dc[t] * (double)ur[q];
                            }
                            dw[ch * 3 + j] += s;
                        }
                    }
                }
            }
            free(buf);
        }
    }
    free(tab);
    return failed ? -1 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
