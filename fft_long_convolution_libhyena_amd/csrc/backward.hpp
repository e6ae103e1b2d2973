// Internal launch interface of the backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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
};

// Bytes of backward workspace for batch B: per (b, d) row the N-1 product
// spectra, the gated-input spectra of steps 0..N-3 and the values v_1..v_{N-2}
// (float2), then the per-row tap sums of the short conv (3 floats per channel).
inline size_t bwd_ws_bytes(int64_t B, int64_t D, int64_t L, int N) {
    const int64_t per_row = (int64_t)(2 * N - 3) * L + (int64_t)(N - 2) * (L / 2);
    return (size_t)(B * D * per_row) * 8 + (size_t)(B * (N + 1) * D * 3) * 4;
}

hipError_t launch_lds_backward(int logL, const LdsBwdArgs& a, hipStream_t st);

}  // namespace hy
