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
    float2* ws;           // bwd_ws_per_channel(L, N) float2 per channel
    const float2* tw;     // Stockham twiddles for length L
    const float2* wpair;  // W_{2L}^k, k = 0..L/2
    int B, D, N;
    bool bf16;
};

// float2 values of backward workspace per channel: the N-1 running dh spectra,
// the unpacked gated-input spectra of steps 0..N-3 and the values v_1..v_{N-2}.
inline int64_t bwd_ws_per_channel(int64_t L, int N) {
    return (int64_t)(2 * N - 3) * L + (int64_t)(N - 2) * (L / 2);
}

hipError_t launch_lds_backward(int logL, const LdsBwdArgs& a, hipStream_t st);

}  // namespace hy
