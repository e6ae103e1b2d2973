// Input-dependent kernel synthesis for gfx950 (HyenaND summary, method:
// input-dependent kernels through registers and FiLM; kernel synthesis; kernel
// parametrisation). Per sample b with control vector z_b, every output kernel k
// at every grid coordinate c is
//   K[b][k](c) = w_k(c) * f_k(c; z_b),
// f a coordinate sine-representation network whose layers are modulated by FiLM:
//   h_0 = c;  h_{l+1} = sin(omega_l * (gamma_l * (W_l h_l + b_l) + beta_l)),
//   gamma_l = G_l z_b + g_l,  beta_l = E_l z_b + e_l;
//   f = W_out h_M + b_out,
// and w_k the axis-aligned Gaussian window exp(-1/2 sum_i ((c_i - mu_ki) / sigma_ki)^2).
// Readings where the summary gives no formula: a sine frequency per hidden unit,
// FiLM on the pre-activation inside the sine, an affine output layer, one window
// per output kernel, causal axes at c = j/n and signed axes at the wrapped offsets
// (j below n/2, j - n above) scaled to [-1, 1). z_b is given per sample: the
// register tokens and their pooling belong to the model around the operator.
//
// The output feeds hyena_filter_spectrum_batched (1-D: C = (N-1)*D kernels on a
// causal axis of L points) and hyena_filter_spectrum{2d,3d}_batched (C = D kernels
// on the signed doubled or periodic grid).
//
// One lane per grid point; a workgroup of four waves covers 64 consecutive points
// of one sample and a block of output kernels. The FiLM vectors of the sample are
// computed once per workgroup into LDS; the hidden stack is evaluated once per
// workgroup (wave w computes units w, w+4, ...; a barrier per layer); then each wave
// takes every fourth output kernel with the final hidden vector of its point in
// registers and the kernel's weights read through the scalar unit.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/hyena.h"
#include "plan.hpp"

namespace hy {
namespace {

constexpr int kSynTile = 64;          // grid points per workgroup, one per lane
constexpr int kSynWaves = 4;          // waves per workgroup, sharing the tile
constexpr int kSynTargetWgs = 4096;   // workgroups to aim for when splitting the kernels
constexpr int kSynMinChans = 64;      // kernels per block otherwise (bounds the stack's re-evaluation)
constexpr int kSynMaxLayers = 16;
constexpr int kSynMaxZ = 256;

struct SynArgs {
    const float* w_first;
    const float* w_hidden;
    const float* b_layer;
    const float* omega;
    const float* film_g;
    const float* film_gb;
    const float* film_b;
    const float* film_bb;
    const float* w_out;
    const float* b_out;
    const float* mu;
    const float* sigma;
    const float* z;
    float* k;
    int64_t n[3];    // points per axis (1 for absent axes)
    int64_t P;       // points per kernel
    int64_t C;       // kernels per sample
    int64_t cpb;     // kernels per workgroup block
    int A, M, Z;
    uint32_t sgn;    // bit i: axis i signed
};

template <int W>
__global__ void __launch_bounds__(kSynTile * kSynWaves) k_kernel_synthesis(SynArgs a) {
    __shared__ float hbuf[2][W * kSynTile];
    __shared__ float film[2][kSynMaxLayers * W];  // gamma, beta of every layer for this sample
    const int lane = threadIdx.x % kSynTile;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kSynTile);
    const int64_t b = blockIdx.z;
    const float* zb = a.z + b * a.Z;

    // FiLM vectors of sample b: gamma = G z + g, beta = E z + e for every layer and unit
#pragma unroll 1
    for (int q = threadIdx.x; q < 2 * a.M * W; q += kSynTile * kSynWaves) {
        const int which = q / (a.M * W), lu = q - which * a.M * W;  // lu = l*W + u
        const float* G = (which == 0 ? a.film_g : a.film_b) + (int64_t)lu * a.Z;
        float acc = (which == 0 ? a.film_gb : a.film_bb)[lu];
#pragma unroll 1
        for (int j = 0; j < a.Z; ++j) acc = fmaf(G[j], zb[j], acc);
        film[which][lu] = acc;
    }

    // this lane's grid point; lanes past the end repeat the last point (they write
    // the same value to the same place, and every lane stays on one path)
    const int64_t p0 = (int64_t)blockIdx.x * kSynTile + lane;
    const int64_t p = p0 < a.P ? p0 : a.P - 1;
    float c[3];
    {
        int64_t rem = p;
#pragma unroll
        for (int i = 2; i >= 0; --i) {
            const int64_t n = a.n[i];  // absent axes have one point
            const int64_t j = rem % n;
            rem /= n;
            const bool sg = (a.sgn >> i) & 1;
            const int64_t off = sg && j >= n / 2 ? j - n : j;
            c[i] = (float)((double)off * ((sg ? 2.0 : 1.0) / (double)n));  // rounded once; 0 on absent axes
        }
    }
    __syncthreads();

    float* cur = hbuf[0];
    float* nxt = hbuf[1];
    // layer 0 from the coordinates
#pragma unroll 1
    for (int u = wave; u < W; u += kSynWaves) {
        float acc = a.b_layer[u];
#pragma unroll
        for (int i = 0; i < 3; ++i)
            if (i < a.A) acc = fmaf(a.w_first[u * a.A + i], c[i], acc);
        cur[u * kSynTile + lane] = sinf(a.omega[u] * fmaf(film[0][u], acc, film[1][u]));
    }
    __syncthreads();
    // hidden layers 1 .. M-1
#pragma unroll 1
    for (int l = 1; l < a.M; ++l) {
        const float* Wl = a.w_hidden + (int64_t)(l - 1) * W * W;
#pragma unroll 1
        for (int u = wave; u < W; u += kSynWaves) {
            float acc = a.b_layer[l * W + u];
#pragma unroll 8
            for (int v = 0; v < W; ++v) acc = fmaf(Wl[u * W + v], cur[v * kSynTile + lane], acc);
            nxt[u * kSynTile + lane] = sinf(a.omega[l * W + u] * fmaf(film[0][l * W + u], acc, film[1][l * W + u]));
        }
        __syncthreads();
        float* t = cur;
        cur = nxt;
        nxt = t;
    }

    // output layer and window: kernel k of this block, at k[b][k][p]
    float r[W];
#pragma unroll
    for (int i = 0; i < W; ++i) r[i] = cur[i * kSynTile + lane];
    const int64_t k0 = (int64_t)blockIdx.y * a.cpb;
    const int64_t k1 = k0 + a.cpb < a.C ? k0 + a.cpb : a.C;
    float* kb = a.k + b * a.C * a.P;
    for (int64_t kk = k0 + wave; kk < k1; kk += kSynWaves) {
        const int kc = __builtin_amdgcn_readfirstlane((int)kk);  // uniform: weights through the scalar unit
        const float* wr = a.w_out + (int64_t)kc * W;
        float f = a.b_out[kc];
#pragma unroll
        for (int i = 0; i < W; ++i) f = fmaf(wr[i], r[i], f);
        float e = 0.f;
#pragma unroll
        for (int i = 0; i < 3; ++i)
            if (i < a.A) {
                const float d = (c[i] - a.mu[kc * a.A + i]) / a.sigma[kc * a.A + i];
                e = fmaf(d, d, e);
            }
        // exp(-e/2) = 2^(-e/2 * log2 e) with the hardware exp2
        const float win = __builtin_amdgcn_exp2f(e * -0.72134752044448170368f);
        kb[(int64_t)kc * a.P + p] = f * win;
    }
}

template <int W>
hipError_t launch_synthesis_t(SynArgs a, int64_t B, hipStream_t st) {
    const int64_t gx = (a.P + kSynTile - 1) / kSynTile;
    // split the kernels only as far as needed to fill the device
    int64_t gy = (kSynTargetWgs + gx * B - 1) / (gx * B);
    int64_t maxy = (a.C + kSynMinChans - 1) / kSynMinChans;
    const int64_t maxw = (a.C + kSynWaves - 1) / kSynWaves;  // at least one kernel per wave
    if (maxy < 1) maxy = 1;
    if (maxy > maxw) maxy = maxw;
    if (gy > maxy) gy = maxy;
    if (gy < 1) gy = 1;
    if (gy > 65535) gy = 65535;
    a.cpb = (a.C + gy - 1) / gy;
    gy = (a.C + a.cpb - 1) / a.cpb;
    hipLaunchKernelGGL((k_kernel_synthesis<W>), dim3((unsigned)gx, (unsigned)gy, (unsigned)B),
                       dim3(kSynTile * kSynWaves), 0, st, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace hy

extern "C" {

hyena_status_t hyena_kernel_synthesis(const hyena_synth_params_t* params, int64_t B, const float* z, float* k,
                                      hipStream_t stream) {
    using hy::aligned16;
    if (!params || !z || !k || B < 1) return HYENA_ERR_INVALID_ARG;
    const hyena_synth_params_t& p = *params;
    if (p.axes < 1 || p.axes > 3 || p.width < 1 || p.layers < 1 || p.zdim < 1 || p.channels < 1)
        return HYENA_ERR_INVALID_ARG;
    int64_t P = 1;
    for (int i = 0; i < p.axes; ++i) {
        if (p.grid[i] < 1) return HYENA_ERR_INVALID_ARG;
        P *= p.grid[i];
        if (P > (int64_t(1) << 28)) return HYENA_ERR_UNSUPPORTED;
    }
    if (p.signed_axes >> p.axes) return HYENA_ERR_INVALID_ARG;
    const float* req[] = {p.w_first, p.b_layer, p.omega, p.film_g, p.film_gb, p.film_b, p.film_bb,
                          p.w_out, p.b_out, p.win_mu, p.win_sigma};
    for (const float* q : req)
        if (!q || !aligned16(q)) return HYENA_ERR_INVALID_ARG;
    if (p.layers > 1 && (!p.w_hidden || !aligned16(p.w_hidden))) return HYENA_ERR_INVALID_ARG;
    if (!aligned16(z) || !aligned16(k)) return HYENA_ERR_INVALID_ARG;
    if (p.layers > hy::kSynMaxLayers || p.zdim > hy::kSynMaxZ) return HYENA_ERR_UNSUPPORTED;
    if (p.width != 8 && p.width != 16 && p.width != 32 && p.width != 64) return HYENA_ERR_UNSUPPORTED;
    if (B > 65535 || p.channels > (int64_t(1) << 24) || (P + hy::kSynTile - 1) / hy::kSynTile > 0x7fffffff)
        return HYENA_ERR_UNSUPPORTED;
    hy::SynArgs a{p.w_first, p.w_hidden, p.b_layer, p.omega, p.film_g, p.film_gb, p.film_b, p.film_bb,
                  p.w_out, p.b_out, p.win_mu, p.win_sigma, z, k, {1, 1, 1}, P, p.channels, 0,
                  (int)p.axes, (int)p.layers, (int)p.zdim, p.signed_axes};
    for (int i = 0; i < p.axes; ++i) a.n[i] = p.grid[i];
    hipError_t e;
    switch (p.width) {
        case 8: e = hy::launch_synthesis_t<8>(a, B, stream); break;
        case 16: e = hy::launch_synthesis_t<16>(a, B, stream); break;
        case 32: e = hy::launch_synthesis_t<32>(a, B, stream); break;
        case 64: e = hy::launch_synthesis_t<64>(a, B, stream); break;
        default: return HYENA_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? HYENA_OK : HYENA_ERR_DEVICE;
}

}  // extern "C"
