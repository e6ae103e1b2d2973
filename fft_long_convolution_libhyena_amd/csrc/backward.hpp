// Internal launch interface of the backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace hy {

struct LdsBwdArgs {
    const void* u;
    const float* w3;
    const float2* spec;
    const float* bias;
    const void* dy;
    void* du;
    float* dw;
    float* dh;
    float* dbias;
    float2* ws;           // bwd_ws_bytes(B, D, L, N) bytes
    const float2* tw;     // Stockham twiddles for length L
    const float2* wpair;  // W_{2L}^k, k = 0..L/2
    int B, D, N;
    bool bf16;
    int64_t sbs = 0;          // spectrum batch stride (complex values): 0 = one spectrum for every b
    bool per_sample = false;  // dh per sample ([B][N-1][D][L]) instead of the batch sum
    bool circ = false;        // circular plan: rows of 2L samples, no zero padding
};

// Bytes of backward workspace for batch B and transform length L: per (b, d) row
// the N-1 product spectra, the gated-input spectra of steps 0..N-3 and the values
// v_1..v_{N-2} (float2; L/2 pairs per value, L for the 2L-sample rows of a
// circular plan), then the per-row tap sums of the short conv (3 floats per channel).
inline size_t bwd_ws_bytes(int64_t B, int64_t D, int64_t L, int N, bool circ = false) {
    const int64_t per_row = (int64_t)(2 * N - 3) * L + (int64_t)(N - 2) * (circ ? L : L / 2);
    return (size_t)(B * D * per_row) * 8 + (size_t)(B * (N + 1) * D * 3) * 4;
}

hipError_t launch_lds_backward(int logL, const LdsBwdArgs& a, hipStream_t st);

// Four-step backward (order 2): arguments and the workspace it carves.
struct FsBwdArgs {
    const void* u;
    const float* w3;
    const float2* spec;
    const float* bias;
    const void* dy;
    void* du;
    float* dw;
    float* dh;
    float* dbias;
    void* ws;  // fs_bwd_ws_bytes(logL, B, D, N, per_sample) bytes
    FsTables tb;
    int B, D, N;
    bool bf16;
    int64_t sbs = 0;          // spectrum batch stride (complex values): 0 = one spectrum for every b
    bool per_sample = false;  // dh per sample ([B][N-1][D][L]) instead of the batch sum
};

// Per (b, d) row: the L-point tile T, the column-transformed gated inputs G_o of
// the N-1 steps and the row's dh tile Tdh (the inverse rows of A_dv * conj(A_g);
// complex),
// the recomputed values v_1..v_{N-2} V (fp32), the N+1 channels' staging rows S
// (fp32), the tap sums of every column-block workgroup; with a filter set per
// sample also every row's lag-0 value. 256-byte aligned.
struct FsBwdWs {
    float2* T;
    float2* G;
    float* V;
    float* S;
    float2* Tdh;
    float* part;
    float* lag;
    size_t bytes;
};
inline FsBwdWs fs_bwd_ws(void* base, int64_t B, int64_t D, int64_t L, int ncb, int N, bool per_sample = false) {
    size_t off = 0;
    auto take = [&](size_t n) {
        void* r = base ? static_cast<char*>(base) + off : nullptr;
        off += (n + 255) & ~(size_t)255;
        return r;
    };
    const size_t rows = (size_t)(B * D);
    FsBwdWs w;
    w.T = (float2*)take(rows * (size_t)L * 8);
    w.G = (float2*)take((size_t)(N - 1) * rows * (size_t)L * 8);
    w.Tdh = (float2*)take(rows * (size_t)L * 8);
    w.V = (float*)take((size_t)(N > 2 ? N - 2 : 0) * rows * (size_t)L * 4);
    w.S = (float*)take(rows * (size_t)(N + 1) * (size_t)L * 4);
    w.part = (float*)take(rows * (size_t)ncb * 3 * (size_t)(N + 1) * 4);
    w.lag = per_sample ? (float*)take(rows * 4) : nullptr;
    w.bytes = off;
    return w;
}
hipError_t launch_fs_backward(int logL, const FsBwdArgs& a, hipStream_t st);
size_t fs_bwd_ws_bytes(int logL, int64_t B, int64_t D, int N, bool per_sample = false);

}  // namespace hy
