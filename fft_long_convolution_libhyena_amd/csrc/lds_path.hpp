// LDS-resident path of the Hyena forward hot path for gfx950 (see kernels.hpp
// for the interface). Explicit instantiations live in lds_path_*.hip.
//
// What is computed (HyenaDNA walkthrough, section 2.1, HyenaOperator.forward;
// section 2.2, HyenaFilter.forward and its fftconv call): a causal width-3
// depthwise conv of every u_proj channel, a split into gates x_0..x_{N-1} and
// the value v, then for o = 0..N-2: v <- v * x_{N-1-o}; v <- conv(v, h[o]) +
// bias[o] * v; finally y = v * x_0. The long convolution is evaluated in the
// frequency domain of a transform of length 2L (zero padding to double length,
// as in the HyenaND summary's boundary handling), which the FFT makes
// O(L log L) (Hyena Hierarchy concept page, section 3.2, FFT acceleration).
//
// Real 2L-point transforms are carried as L-point complex transforms of the
// packed sequence z[m] = a[2m] + i a[2m+1]. The second half of z is the zero
// padding (never loaded, pruned in the first radix pass), and only the first
// half of the inverse is kept. Bins k and L-k are combined in one "pair step"
// that unpacks the forward spectrum, multiplies by the filter spectrum plus the
// bias (the skip term bias*v is the convolution of v with bias*delta, whose
// spectrum is the constant bias) and repacks for the inverse. The stored
// filter spectrum is scaled by 2^-(log2 L + 2) (exact) so that the pair step
// also applies the inverse normalisation.
//
// Two paths:
//  * LDS path (L <= 16384): one workgroup per (b, d) row keeps the whole
//    transform on chip for all N-1 steps; only u_proj, the spectrum and y touch
//    HBM.
//  * Four-step path (any L >= 256, used for L >= 32768): L = L1 * L2 with
//    m = L2*m1 + m2 and k = k1 + L1*k2. Pass A takes column FFTs over m1,
//    pass B takes row FFTs over m2 (with the L-point twiddle), the pair step and
//    the inverse rows, pass C takes the inverse columns and the gate. Pass C of
//    step o is fused with pass A of step o+1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "kernels.hpp"
#include "pair.hpp"

namespace hy {

// =================================================================== LDS path

// N (the recurrence order) is a template parameter so the step loop unrolls:
// with a run-time trip count the compiler keeps both transforms' state live
// across the loop and needs about twice the registers.
// CIRC: circular convolution of sequences of 2L samples (the HyenaND summary's
// circular boundary mode): the same L-point packed transform with every slot
// holding data (no zero-padded half, no pruned first pass) and every output kept.
// At order 2 the register budget is the one that keeps every workgroup the LDS
// allows resident (it fits without spills); higher orders keep more state live
// across the step loop and get the compiler's default.
template <int LOGL, int N, class TIO, bool CIRC = false>
__global__ void __launch_bounds__(LdsCfg<LOGL>::THREADS, N == 2 ? LdsCfg<LOGL>::MIN_WAVES : 1)
k_lds_forward(const TIO* __restrict__ u, const float* __restrict__ w3, const float2* __restrict__ spec,
              const float* __restrict__ bias, TIO* __restrict__ y, const float2* __restrict__ tw,
              const float2* __restrict__ wpair, int B, int D, int64_t sbs) {
    constexpr int L = 1 << LOGL;
    constexpr int E = LdsCfg<LOGL>::E;
    constexpr int H = E / 2;
    constexpr int T = L / E;
    constexpr int64_t S = CIRC ? 2 * (int64_t)L : L;  // samples per row of u_proj and y
    constexpr int LD = CIRC ? E : H;                  // slots holding data
    constexpr bool PF_GATE = HY_LDS_PREFETCH_GATE && !CIRC;
    __shared__ float2 lds[padded_len<L>()];
    const RowAcc acc{lds};
    // Consecutive workgroups go to different XCDs; the B batch rows of channel d
    // are given to workgroups of one XCD so that its L2 serves the shared spectrum.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, s = bid >> 3;
    const int b = s % B;
    const int d = (s / B) * 8 + xcd;
    if (d >= D) return;
    const int t = threadIdx.x;
    const int64_t C = (int64_t)(N + 1) * D;
    const TIO* ub = u + (int64_t)b * C * S;

    float2 v[E];
    {
        const int cv = N * D + d, cx = (N - 1) * D + d;
        const TIO* rv = ub + (int64_t)cv * S;
        const TIO* rx = ub + (int64_t)cx * S;
#pragma unroll
        for (int e = 0; e < LD; ++e) v[e] = gated_pair(rv, rx, (uint32_t)(t + T * e), w3 + 3 * cv, w3 + 3 * cx);
#pragma unroll
        for (int e = LD; e < E; ++e) v[e] = make_float2(0.f, 0.f);
    }
    const float bscale = 1.0f / (4.0f * (float)L);
#pragma unroll
    for (int o = 0; o < N - 1; ++o) {
        // keep each step's loads inside its step: hoisting the next step's
        // spectrum fetch across a transform raises register pressure
        __builtin_amdgcn_sched_barrier(0);
        const float2* Hs = spec + (int64_t)b * sbs + ((int64_t)o * D + d) * L;
        // spectrum values of this thread's pairs, fetched before the transform
        float2 hk[H], hm[H];
        if constexpr (HY_LDS_PREFETCH) {
#pragma unroll
            for (int e = 0; e < H; ++e) {
                const uint32_t k = t + T * e;
                hk[e] = ld32(Hs, k);
                hm[e] = ld32(Hs, k == 0 ? 0u : (uint32_t)L - k);
            }
        }
        fft_strided<L, false, !CIRC>(v, t, tw, acc);
        __syncthreads();
        lds_store_strided<T>(acc, t, v);
        __syncthreads();
        const float bs = bias[o * D + d] * bscale;
#pragma unroll
        for (int e = 0; e < H; ++e) {
            const uint32_t k = t + T * e;  // k in [0, L/2)
            const uint32_t km = k == 0 ? 0 : L - k;
            if constexpr (!HY_LDS_PREFETCH) {
                hk[e] = ld32(Hs, k);
                hm[e] = ld32(Hs, km);
            }
            float2 Hk, Hm;
            if (k == 0) {
                Hk = make_float2(hk[e].x + bs, 0.f);
                Hm = make_float2(hk[e].y + bs, 0.f);
            } else {
                Hk = hadd(hk[e], bs);
                Hm = hadd(hm[e], bs);
            }
            float2 Yk, Ym;
            pair_conv(acc[k], acc[km], Hk, Hm, ld32(wpair, k), Yk, Ym);
            acc[k] = Yk;
            if (k != 0) acc[km] = Ym;
        }
        if (t == 0) {  // k = L/2 pairs with itself
            const uint32_t k = L / 2;
            const float2 Hk = hadd(Hs[k], bs);
            float2 Yk, Ym;
            const float2 Z = acc[k];
            pair_conv(Z, Z, Hk, Hk, wpair[k], Yk, Ym);
            acc[k] = Yk;
        }
        __syncthreads();
        lds_load_strided<T>(acc, t, v);
        const bool last = (o == N - 2);
        const int cg = (last ? 0 : N - 2 - o) * D + d;
        const TIO* rg = ub + (int64_t)cg * S;
        const float* wg = w3 + 3 * cg;
        // the gate's input samples, fetched before the inverse transform so that
        // their latency hides behind it
        typename RawPair<TIO>::type gcur[H], gprev[H];
        if constexpr (PF_GATE) {
            if (last) {
#pragma unroll
                for (int e = 0; e < H; ++e) {
                    const uint32_t m = t + T * e;
                    gcur[e] = load_raw(rg, m);
                    gprev[e] = m > 0 ? load_raw(rg, m - 1) : RawPair<TIO>::zero();
                }
            }
        }
        fft_strided<L, true, false>(v, t, tw, acc);
        // v[e], e < E/2, holds (c[2m], c[2m+1]) = conv + bias*v at m = t + T*e
        if (last) {
            TIO* yr = y + ((int64_t)b * D + d) * S;
#pragma unroll
            for (int e = 0; e < LD; ++e) {
                const uint32_t m = t + T * e;
                float2 g;
                if constexpr (PF_GATE)
                    g = conv3_from(unpack_raw(gprev[e]), unpack_raw(gcur[e]), wg[0], wg[1], wg[2]);
                else
                    g = conv3_pair(rg, m, wg[0], wg[1], wg[2]);
                store_pair(yr, m, emul(v[e], g));
            }
        } else {
#pragma unroll
            for (int e = 0; e < LD; ++e) v[e] = emul(v[e], conv3_pair(rg, (uint32_t)(t + T * e), wg[0], wg[1], wg[2]));
#pragma unroll
            for (int e = LD; e < E; ++e) v[e] = make_float2(0.f, 0.f);
        }
    }
}

// Filter spectrum for the LDS path: natural-order bins, slot 0 = (A[0], A[L]),
// every value scaled by 1/(4L).
// CIRC: the filter has 2L samples and no zero padding (circular mode).
template <int LOGL, bool CIRC = false>
__global__ void __launch_bounds__(LdsCfg<LOGL>::THREADS)
k_lds_spectrum(const float* __restrict__ h, float2* __restrict__ spec, const float2* __restrict__ tw,
               const float2* __restrict__ wpair) {
    constexpr int L = 1 << LOGL;
    constexpr int E = LdsCfg<LOGL>::E;
    constexpr int H = E / 2;
    constexpr int T = L / E;
    constexpr int64_t S = CIRC ? 2 * (int64_t)L : L;
    constexpr int LD = CIRC ? E : H;
    __shared__ float2 lds[padded_len<L>()];
    const RowAcc acc{lds};
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const float* hr = h + row * S;
    float2* out = spec + row * L;
    float2 v[E];
#pragma unroll
    for (int e = 0; e < LD; ++e) v[e] = load_pair(hr, (uint32_t)(t + T * e));
#pragma unroll
    for (int e = LD; e < E; ++e) v[e] = make_float2(0.f, 0.f);
    fft_strided<L, false, !CIRC>(v, t, tw, acc);
    __syncthreads();
    lds_store_strided<T>(acc, t, v);
    __syncthreads();
    const float sc = 1.0f / (8.0f * (float)L);  // (2A) / (8L) = A / (4L)
#pragma unroll
    for (int e = 0; e < H; ++e) {
        const uint32_t k = t + T * e;
        const uint32_t km = k == 0 ? 0 : L - k;
        float2 Ak, Am;
        pair_unpack(acc[k], acc[km], wpair[k], Ak, Am);
        if (k == 0) {
            out[0] = make_float2(Ak.x * sc, Am.x * sc);
        } else {
            out[k] = fmul2(Ak, sc);
            out[km] = fmul2(Am, sc);
        }
    }
    if (t == 0) {
        const uint32_t k = L / 2;
        float2 Ak, Am;
        const float2 Z = acc[k];
        pair_unpack(Z, Z, wpair[k], Ak, Am);
        out[k] = fmul2(Ak, sc);
    }
}

template <int LOGL, int N, bool CIRC>
inline void launch_lds_forward_c(const LdsArgs& a, hipStream_t st) {
    constexpr int T = LdsCfg<LOGL>::THREADS;
    const int dgroups = (a.D + 7) / 8;
    const unsigned grid = (unsigned)(a.B * 8 * dgroups);
    if (a.bf16)
        hipLaunchKernelGGL((k_lds_forward<LOGL, N, uint16_t, CIRC>), dim3(grid), dim3(T), 0, st,
                           (const uint16_t*)a.u, a.w3, a.spec, a.bias, (uint16_t*)a.y, a.tw, a.wpair, a.B, a.D,
                           a.sbs);
    else
        hipLaunchKernelGGL((k_lds_forward<LOGL, N, float, CIRC>), dim3(grid), dim3(T), 0, st, (const float*)a.u,
                           a.w3, a.spec, a.bias, (float*)a.y, a.tw, a.wpair, a.B, a.D, a.sbs);
}

template <int LOGL, int N>
inline void launch_lds_forward_n(const LdsArgs& a, hipStream_t st) {
    if (a.circ)
        launch_lds_forward_c<LOGL, N, true>(a, st);
    else
        launch_lds_forward_c<LOGL, N, false>(a, st);
}

template <int LOGL>
hipError_t launch_lds_forward_t(const LdsArgs& a, hipStream_t st) {
    switch (a.N) {
        case 2: launch_lds_forward_n<LOGL, 2>(a, st); break;
        case 3: launch_lds_forward_n<LOGL, 3>(a, st); break;
        case 4: launch_lds_forward_n<LOGL, 4>(a, st); break;
        case 5: launch_lds_forward_n<LOGL, 5>(a, st); break;
        case 6: launch_lds_forward_n<LOGL, 6>(a, st); break;
        case 7: launch_lds_forward_n<LOGL, 7>(a, st); break;
        case 8: launch_lds_forward_n<LOGL, 8>(a, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int LOGL>
hipError_t launch_lds_spectrum_t(const float* h, float2* spec, int64_t rows, const float2* tw,
                                        const float2* wpair, hipStream_t st, bool circ) {
    if (circ)
        hipLaunchKernelGGL((k_lds_spectrum<LOGL, true>), dim3((unsigned)rows), dim3(LdsCfg<LOGL>::THREADS), 0, st,
                           h, spec, tw, wpair);
    else
        hipLaunchKernelGGL((k_lds_spectrum<LOGL, false>), dim3((unsigned)rows), dim3(LdsCfg<LOGL>::THREADS), 0,
                           st, h, spec, tw, wpair);
    return hipGetLastError();
}

}  // namespace hy
