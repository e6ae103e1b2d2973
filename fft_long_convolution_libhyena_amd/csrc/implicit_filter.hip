// Implicit long-filter generator for gfx950 (HyenaDNA walkthrough, section 2.2,
// HyenaFilter.filter and its constructor): the positional features of every time
// step, a Linear(emb_dim -> W) / Sin stack with num_inner further Linear(W -> W) /
// Sin layers, a Linear(W -> (N-1)*D) without bias, the exponential modulation, and
// the [L, (N-1)*D] -> [N-1][D][L] reshape of section 2.1, written straight into the
// h[o][d][t] layout that hyena_filter_spectrum reads.
//
// Readings where the pages give no formula: t = tau / L; the features are
// (t, sin(2 pi f_k t) for the K = (emb_dim-1)/2 bands, then cos(2 pi f_k t)) with
// the band frequencies f_k an input; Sin(x) = sin(freq * x) elementwise with one
// frequency vector shared by every Sin of the stack (the walkthrough's code appends
// the same activation module after each Linear); the modulation multiplies channel
// c by exp(-alpha_c * t), evaluated as 2^(alpha_c * (-t log2 e)) with the hardware
// exp2 (about 1e-7 relative error, mostly from rounding the argument; arguments
// stay far above the exponent range where its result would flush to zero for any
// |alpha| * t below 80).
//
// One lane per time step; a workgroup of four waves covers 64 consecutive steps
// and a block of output channels, so each output row segment it writes is 256
// bytes of consecutive time steps. The weights are the same for every thread and are read
// through the scalar unit. The positional features are evaluated in fp64 and
// rounded once; the stack runs in fp32 with the device's accurate sinf.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/hyena.h"
#include "plan.hpp"

namespace hy {
namespace {

constexpr int kFiltTile = 64;         // time steps per workgroup, one per lane
constexpr int kFiltWaves = 4;         // waves per workgroup, sharing the tile
constexpr int kFiltTargetWgs = 4096;  // workgroups to aim for when splitting the channels
constexpr int kFiltMinWgs = 1024;     // below this, blocks may hold fewer channels
constexpr int kFiltMinChans = 64;     // channels per block otherwise (bounds the stack's re-evaluation)
constexpr int kMaxEmbDim = 127;
constexpr int kMaxInner = 16;

// The four waves of a workgroup serve the same 64 time steps (lane = step). The
// hidden vector of step `lane` lives in LDS (unit j at j*64 + lane); in every layer
// wave w computes units w, w+4, w+8, ... from all of the previous layer's units,
// with a barrier between layers, so the stack is evaluated once per workgroup. The
// waves then take every fourth output channel of the workgroup's block, with the
// final hidden vector of their step in registers.
template <int W>
__global__ void __launch_bounds__(kFiltTile * kFiltWaves)
k_implicit_filter(const float* __restrict__ band, const float* __restrict__ w_in, const float* __restrict__ b_in,
                  const float* __restrict__ w_inner, const float* __restrict__ b_inner,
                  const float* __restrict__ sfreq, const float* __restrict__ w_out, const float* __restrict__ alpha,
                  float* __restrict__ h, int E, int M, int64_t C, int64_t cpb, int logL) {
    __shared__ float buf[2][W * kFiltTile];
    const int lane = threadIdx.x % kFiltTile;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kFiltTile);
    const int64_t L = int64_t(1) << logL;
    // lanes past the end (L < 64) repeat step L-1: they write the same value to the
    // same place, and every lane stays on one branch-free path
    const int64_t tau0 = (int64_t)blockIdx.x * kFiltTile + lane;
    const int64_t tau = tau0 < L ? tau0 : L - 1;
    const double td = ldexp((double)tau, -logL);
    const float t = (float)td;  // exact: tau < 2^24
    float* a = buf[0];
    float* b = buf[1];

    // Linear(E -> W) on the positional features, then Sin: this wave's units
    const int K = (E - 1) / 2;
#pragma unroll 1
    for (int j = wave; j < W; j += kFiltWaves) a[j * kFiltTile + lane] = fmaf(w_in[j * E], t, b_in[j]);
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
        double sd, cd;
        sincos(2.0 * M_PI * (double)band[k] * td, &sd, &cd);
        const float zs = (float)sd, zc = (float)cd;
#pragma unroll 1
        for (int j = wave; j < W; j += kFiltWaves) {
            float* q = a + j * kFiltTile + lane;
            *q = fmaf(w_in[j * E + 1 + K + k], zc, fmaf(w_in[j * E + 1 + k], zs, *q));
        }
    }
#pragma unroll 1
    for (int j = wave; j < W; j += kFiltWaves) a[j * kFiltTile + lane] = sinf(sfreq[j] * a[j * kFiltTile + lane]);
    __syncthreads();

    // inner Linear(W -> W) + Sin layers
#pragma unroll 1
    for (int m = 0; m < M; ++m) {
        const float* wm = w_inner + (int64_t)m * W * W;
        const float* bm = b_inner + (int64_t)m * W;
#pragma unroll 1
        for (int j = wave; j < W; j += kFiltWaves) {
            float acc = bm[j];
#pragma unroll 8
            for (int i = 0; i < W; ++i) acc = fmaf(wm[j * W + i], a[i * kFiltTile + lane], acc);
            b[j * kFiltTile + lane] = sinf(sfreq[j] * acc);
        }
        __syncthreads();
        float* tmp = a;
        a = b;
        b = tmp;
    }

    // output Linear without bias, modulation, channel c = o*D + d at h[c][tau]
    float r[W];
#pragma unroll
    for (int i = 0; i < W; ++i) r[i] = a[i * kFiltTile + lane];
    // exp(-alpha t) = 2^(alpha * (-t log2 e)): one product and the hardware exp2
    const float tn = (float)(-td * 1.4426950408889634);
    const int c0 = (int)(blockIdx.y * cpb);
    const int c1 = (int)(c0 + cpb < C ? c0 + cpb : C);
#pragma unroll 2
    for (int cc = c0 + wave; cc < c1; cc += kFiltWaves) {
        const int c = __builtin_amdgcn_readfirstlane(cc);  // uniform: the weights come through the scalar unit
        const float* wr = w_out + (int64_t)c * W;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < W; ++i) acc = fmaf(wr[i], r[i], acc);
        const float v = acc * __builtin_amdgcn_exp2f(alpha[c] * tn);
        (h + ((int64_t)c << logL))[tau] = v;
    }
}

template <int W>
hipError_t launch_filter_t(const hyena_filter_mlp_t& p, float* h, int64_t C, int logL, hipStream_t st) {
    const int64_t L = int64_t(1) << logL;
    const int64_t gx = (L + kFiltTile - 1) / kFiltTile;
    // split the channels only as far as needed to fill the device
    int64_t gy = (kFiltTargetWgs + gx - 1) / gx;
    int64_t maxy = (C + kFiltMinChans - 1) / kFiltMinChans;
    if (gx * maxy < kFiltMinWgs) maxy = (kFiltMinWgs + gx - 1) / gx;
    const int64_t maxw = (C + kFiltWaves - 1) / kFiltWaves;  // at least one channel per wave
    if (maxy > maxw) maxy = maxw;
    if (gy > maxy) gy = maxy;
    if (gy > 65535) gy = 65535;
    const int64_t cpb = (C + gy - 1) / gy;
    gy = (C + cpb - 1) / cpb;
    hipLaunchKernelGGL((k_implicit_filter<W>), dim3((unsigned)gx, (unsigned)gy), dim3(kFiltTile * kFiltWaves), 0,
                       st, p.band_freq, p.w_in, p.b_in, p.w_inner, p.b_inner, p.sin_freq, p.w_out, p.alpha, h,
                       (int)p.emb_dim, (int)p.num_inner, C, cpb, logL);
    return hipGetLastError();
}

}  // namespace
}  // namespace hy

extern "C" {

hyena_status_t hyena_implicit_filter(hyena_plan_t plan, const hyena_filter_mlp_t* mlp, float* h,
                                     hipStream_t stream) {
    using hy::aligned16;
    if (!plan || !mlp || !h) return HYENA_ERR_INVALID_ARG;
    const hyena_filter_mlp_t& p = *mlp;
    if (p.emb_dim < 3 || p.emb_dim % 2 == 0 || p.width < 1 || p.num_inner < 0) return HYENA_ERR_INVALID_ARG;
    if (!p.band_freq || !p.w_in || !p.b_in || !p.sin_freq || !p.w_out || !p.alpha) return HYENA_ERR_INVALID_ARG;
    if (p.num_inner > 0 && (!p.w_inner || !p.b_inner)) return HYENA_ERR_INVALID_ARG;
    const void* ptrs[] = {p.band_freq, p.w_in, p.b_in, p.sin_freq, p.w_out, p.alpha, h};
    for (const void* q : ptrs)
        if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
    if (p.num_inner > 0 && (!aligned16(p.w_inner) || !aligned16(p.b_inner))) return HYENA_ERR_INVALID_ARG;
    if (p.emb_dim > hy::kMaxEmbDim || p.num_inner > hy::kMaxInner) return HYENA_ERR_UNSUPPORTED;
    if (p.width != 8 && p.width != 16 && p.width != 32 && p.width != 64) return HYENA_ERR_UNSUPPORTED;
    if (hy::check_device(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    const int64_t C = (int64_t)(plan->order - 1) * plan->D;
    hipError_t e;
    switch (p.width) {
        case 8: e = hy::launch_filter_t<8>(p, h, C, plan->logL, stream); break;
        case 16: e = hy::launch_filter_t<16>(p, h, C, plan->logL, stream); break;
        case 32: e = hy::launch_filter_t<32>(p, h, C, plan->logL, stream); break;
        case 64: e = hy::launch_filter_t<64>(p, h, C, plan->logL, stream); break;
        default: return HYENA_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? HYENA_OK : HYENA_ERR_DEVICE;
}

}  // extern "C"
