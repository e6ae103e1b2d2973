/*
 * Drives every exported function of the C oracle (oracle/hyena_oracle.c) on small
 * seeded inputs, for a build with the address and undefined-behaviour sanitizers
 * (tests/test_oracle_sanitize.py). It checks no numbers: a sanitizer report or a
 * wrong return code fails the run. Inputs come from a plain 64-bit LCG, which is
 * test data only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_short_conv_row(const float* u, const float* w3, int64_t L, double* out);
void oracle_causal_conv_direct(const double* v, const double* h, int64_t L, double* out);
void oracle_causal_conv_fft(const double* v, const double* h, int64_t L, double* out);
int oracle_fft(double* re, double* im, int64_t n, int sign);
int oracle_hyena_forward(int64_t B, int64_t D, int64_t L, int N, const float* u, const double* u64, const float* w,
                         const float* h, const float* bias, const int64_t* rows, int64_t nrows, double* y, int mode,
                         int nthreads);
void oracle_causal_corr_direct(const double* a, const double* k, int64_t L, double* out);
void oracle_causal_corr_fft(const double* a, const double* k, int64_t L, double* out);
int oracle_hyena_backward(int64_t B, int64_t D, int64_t L, int N, const float* u, const float* w, const float* h,
                          const float* bias, const float* dy, double* du, double* dw, double* dh, double* dbias,
                          int mode, int nthreads);
int oracle_max_threads(void);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double next_value(void) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(state >> 11) * (1.0 / 9007199254740992.0) - 0.5;
}
static float* fvec(int64_t n) {
    float* p = (float*)malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = (float)next_value();
    return p;
}
static double* dvec(int64_t n) {
    double* p = (double*)malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = next_value();
    return p;
}
static int fails = 0;
static void expect(int cond, const char* what) {
    if (!cond) {
        fprintf(stderr, "unexpected result: %s\n", what);
        ++fails;
    }
}

static void run_shape(int64_t B, int64_t D, int64_t L, int N) {
    const int64_t C = (N + 1) * D;
    float* u = fvec(B * C * L);
    float* w = fvec(C * 3);
    float* h = fvec((N - 1) * D * L);
    float* bias = fvec((N - 1) * D);
    float* dy = fvec(B * D * L);
    double* u64 = dvec(B * C * L);
    double* y = dvec((B * D > 2 ? B * D : 2) * L);  // all rows, or the two listed ones
    double* du = dvec(B * C * L);
    double* dw = dvec(C * 3);
    double* dh = dvec((N - 1) * D * L);
    double* db = dvec((N - 1) * D);
    int64_t rows[2] = {0, B * D - 1};
    for (int mode = 0; mode <= 1; ++mode) {
        expect(oracle_hyena_forward(B, D, L, N, u, NULL, w, h, bias, NULL, 0, y, mode, 1) == 0, "forward");
        expect(oracle_hyena_forward(B, D, L, N, NULL, u64, w, h, bias, rows, 2, y, mode, 1) == 0, "forward rows");
        expect(oracle_hyena_backward(B, D, L, N, u, w, h, bias, dy, du, dw, dh, db, mode, 1) == 0, "backward");
    }
    int64_t bad_rows[1] = {B * D};
    expect(oracle_hyena_forward(B, D, L, N, u, NULL, w, h, bias, bad_rows, 1, y, 1, 1) == -1, "row out of range");
    expect(oracle_hyena_forward(B, D, L, 1, u, NULL, w, h, bias, NULL, 0, y, 1, 1) == -1, "order 1");
    expect(oracle_hyena_forward(B, D, L, N, NULL, NULL, w, h, bias, NULL, 0, y, 1, 1) == -1, "no input");
    expect(oracle_hyena_forward(B, D, L, N, u, NULL, w, h, bias, NULL, 0, y, 2, 1) == -1, "bad mode");
    expect(oracle_hyena_backward(B, D, L, N, u, w, h, bias, dy, NULL, dw, dh, db, 1, 1) == -1, "no du");
    free(u); free(w); free(h); free(bias); free(dy); free(u64); free(y); free(du); free(dw); free(dh); free(db);
}

int main(void) {
    const int64_t lens[] = {1, 2, 3, 5, 16, 17, 64, 100};
    for (size_t i = 0; i < sizeof(lens) / sizeof(lens[0]); ++i) {
        const int64_t L = lens[i];
        float* u = fvec(L);
        float* w3 = fvec(3);
        double* a = dvec(L);
        double* k = dvec(L);
        double* o1 = dvec(L);
        double* o2 = dvec(L);
        oracle_short_conv_row(u, w3, L, o1);
        oracle_causal_conv_direct(a, k, L, o1);
        oracle_causal_conv_fft(a, k, L, o2);
        oracle_causal_corr_direct(a, k, L, o1);
        oracle_causal_corr_fft(a, k, L, o2);
        free(u); free(w3); free(a); free(k); free(o1); free(o2);
    }
    for (int64_t n = 1; n <= 256; n *= 2) {
        double* re = dvec(n);
        double* im = dvec(n);
        expect(oracle_fft(re, im, n, -1) == 0 && oracle_fft(re, im, n, +1) == 0, "fft");
        free(re); free(im);
    }
    double re3[3] = {0, 0, 0}, im3[3] = {0, 0, 0};
    expect(oracle_fft(re3, im3, 3, -1) == -1, "fft of length 3");
    run_shape(1, 1, 1, 2);
    run_shape(2, 3, 5, 3);
    run_shape(1, 2, 16, 4);
    run_shape(2, 1, 33, 2);
    expect(oracle_max_threads() >= 1, "threads");
    printf("oracle driver: %d unexpected results\n", fails);
    return fails ? 1 : 0;
}
