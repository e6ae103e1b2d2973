// HIP kernels of the Hyena forward hot path for gfx950.
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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "kernels.hpp"

namespace hy {

// ------------------------------------------------------------------ pair step
//
// Zk = Z[k], Zm = Z[L-k] of the packed L-point forward transform; w = W_{2L}^k.
// Returns 2*A[k] and 2*A[L-k], A being the 2L-point spectrum of the real input:
//   E = (Z[k] + conj Z[L-k]) / 2, O = (Z[k] - conj Z[L-k]) / 2i,
//   A[k] = E + W^k O, A[L-k] = conj(E - W^k O).
__device__ __forceinline__ void pair_unpack(float2 Zk, float2 Zm, float2 w, float2& Ak, float2& Am) {
    const float2 Ep = make_float2(Zk.x + Zm.x, Zk.y - Zm.y);  // Zk + conj(Zm)
    const float2 Dp = make_float2(Zk.x - Zm.x, Zk.y + Zm.y);  // Zk - conj(Zm)
    const float2 Op = make_float2(Dp.y, -Dp.x);                // -i * Dp
    const float2 P = cmul(w, Op);
    Ak = cadd(Ep, P);
    Am = make_float2(Ep.x - P.x, P.y - Ep.y);  // conj(Ep - P)
}

// Spectrum multiply and repack for the inverse. Hk, Hm are the scaled filter
// spectrum plus scaled bias at k and L-k. With C = A*H:
//   Y[k] = Ec + i Oc, Ec = (C[k] + conj C[L-k])/2, Oc = (C[k] - conj C[L-k]) W^-k / 2,
//   Y[L-k] = conj(Ec) + i conj(Oc).
__device__ __forceinline__ void pair_conv(float2 Zk, float2 Zm, float2 Hk, float2 Hm, float2 w, float2& Yk,
                                          float2& Ym) {
    float2 Ak, Am;
    pair_unpack(Zk, Zm, w, Ak, Am);
    const float2 Ck = cmul(Ak, Hk);
    const float2 Cm = cmul(Am, Hm);
    const float2 Ec = make_float2(Ck.x + Cm.x, Ck.y - Cm.y);
    const float2 Dc = make_float2(Ck.x - Cm.x, Ck.y + Cm.y);
    const float2 Oc = cmulc(Dc, w);
    Yk = make_float2(Ec.x - Oc.y, Ec.y + Oc.x);
    Ym = make_float2(Ec.x + Oc.y, Oc.x - Ec.y);
}

__device__ __forceinline__ float2 fmul2(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
__device__ __forceinline__ float2 hadd(float2 h, float b) { return make_float2(h.x + b, h.y); }
__device__ __forceinline__ float2 emul(float2 a, float2 b) { return make_float2(a.x * b.x, a.y * b.y); }

template <class TIO>
__device__ __forceinline__ float2 gated_pair(const TIO* __restrict__ rv, const TIO* __restrict__ rx, int64_t m,
                                             const float* wv, const float* wx) {
    const float2 a = conv3_pair(rv, m, wv[0], wv[1], wv[2]);
    const float2 g = conv3_pair(rx, m, wx[0], wx[1], wx[2]);
    return emul(a, g);
}

// =================================================================== LDS path

template <int LOGL, class TIO>
__global__ void __launch_bounds__(LdsCfg<LOGL>::THREADS)
k_lds_forward(const TIO* __restrict__ u, const float* __restrict__ w3, const float2* __restrict__ spec,
              const float* __restrict__ bias, TIO* __restrict__ y, const float2* __restrict__ tw,
              const float2* __restrict__ wpair, int B, int D, int N) {
    constexpr int L = 1 << LOGL;
    constexpr int T = L / 16;
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
    const TIO* ub = u + (int64_t)b * C * L;

    float2 v[16];
    {
        const int cv = N * D + d, cx = (N - 1) * D + d;
        const TIO* rv = ub + (int64_t)cv * L;
        const TIO* rx = ub + (int64_t)cx * L;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = gated_pair(rv, rx, t + T * e, w3 + 3 * cv, w3 + 3 * cx);
#pragma unroll
        for (int e = 8; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
    }
    const float bscale = 1.0f / (4.0f * (float)L);
    for (int o = 0; o < N - 1; ++o) {
        fft_strided<L, false, true>(v, t, tw, acc);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t + T * e] = v[e];
        __syncthreads();
        const float2* H = spec + ((int64_t)o * D + d) * L;
        const float bs = bias[o * D + d] * bscale;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = t + T * e;  // k in [0, L/2)
            const int km = k == 0 ? 0 : L - k;
            float2 Hk, Hm;
            if (k == 0) {
                const float2 h0 = H[0];
                Hk = make_float2(h0.x + bs, 0.f);
                Hm = make_float2(h0.y + bs, 0.f);
            } else {
                Hk = hadd(H[k], bs);
                Hm = hadd(H[km], bs);
            }
            float2 Yk, Ym;
            pair_conv(acc[k], acc[km], Hk, Hm, wpair[k], Yk, Ym);
            acc[k] = Yk;
            if (k != 0) acc[km] = Ym;
        }
        if (t == 0) {  // k = L/2 pairs with itself
            const int k = L / 2;
            const float2 Hk = hadd(H[k], bs);
            float2 Yk, Ym;
            const float2 Z = acc[k];
            pair_conv(Z, Z, Hk, Hk, wpair[k], Yk, Ym);
            acc[k] = Yk;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = acc[t + T * e];
        fft_strided<L, true, false>(v, t, tw, acc);
        // v[e], e < 8, holds (c[2m], c[2m+1]) = conv + bias*v at m = t + T*e
        const bool last = (o == N - 2);
        const int cg = (last ? 0 : N - 2 - o) * D + d;
        const TIO* rg = ub + (int64_t)cg * L;
        const float* wg = w3 + 3 * cg;
        if (last) {
            TIO* yr = y + ((int64_t)b * D + d) * L;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t m = t + T * e;
                store_pair(yr, m, emul(v[e], conv3_pair(rg, m, wg[0], wg[1], wg[2])));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = emul(v[e], conv3_pair(rg, (int64_t)(t + T * e), wg[0], wg[1], wg[2]));
#pragma unroll
            for (int e = 8; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
        }
    }
}

// Filter spectrum for the LDS path: natural-order bins, slot 0 = (A[0], A[L]),
// every value scaled by 1/(4L).
template <int LOGL>
__global__ void __launch_bounds__(LdsCfg<LOGL>::THREADS)
k_lds_spectrum(const float* __restrict__ h, float2* __restrict__ spec, const float2* __restrict__ tw,
               const float2* __restrict__ wpair) {
    constexpr int L = 1 << LOGL;
    constexpr int T = L / 16;
    __shared__ float2 lds[padded_len<L>()];
    const RowAcc acc{lds};
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const float* hr = h + row * L;
    float2* out = spec + row * L;
    float2 v[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = load_pair(hr, t + T * e);
#pragma unroll
    for (int e = 8; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
    fft_strided<L, false, true>(v, t, tw, acc);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t + T * e] = v[e];
    __syncthreads();
    const float sc = 1.0f / (8.0f * (float)L);  // (2A) / (8L) = A / (4L)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k = t + T * e;
        const int km = k == 0 ? 0 : L - k;
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
        const int k = L / 2;
        float2 Ak, Am;
        const float2 Z = acc[k];
        pair_unpack(Z, Z, wpair[k], Ak, Am);
        out[k] = fmul2(Ak, sc);
    }
}

// ============================================================ four-step path

// W_L^a for 0 <= a < L from two tables: W_L^a = hi[a >> SLO] * lo[a & (2^SLO - 1)].
__device__ __forceinline__ float2 twiddle_L(const FsTables& tb, int a) {
    return cmul(tb.othi[a >> tb.slo], tb.otlo[a & ((1 << tb.slo) - 1)]);
}

// Pass A: column FFTs over m1 of the packed gated input (MODE 0) or of a filter
// row (MODE 1), written to the row-major [k1][m2] tile of the row's slot.
template <int LOG1, int LOG2, class TIO, int MODE>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::COL_THREADS))
k_fs_colfwd(const TIO* __restrict__ u, const float* __restrict__ w3, const float* __restrict__ h,
            float2* __restrict__ ws, FsTables tb, int D, int N, int64_t row0) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T1 = Cfg::T1, CB = Cfg::CB;
    constexpr int64_t L = (int64_t)L1 * L2;
    __shared__ float2 lds[L1 * Cfg::CP];
    const int cb = blockIdx.x % (L2 / CB);
    const int64_t r = blockIdx.x / (L2 / CB);
    const int64_t flat = row0 + r;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m2 = cb * CB + c;
    float2 v[16];
    float2* slot;
    if constexpr (MODE == 0) {
        const int64_t b = flat / D, d = flat % D;
        const int64_t C = (int64_t)(N + 1) * D;
        const int64_t cv = N * D + d, cx = (N - 1) * D + d;
        const TIO* rv = u + (b * C + cv) * L;
        const TIO* rx = u + (b * C + cx) * L;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t m = (int64_t)(t + T1 * e) * L2 + m2;
            v[e] = gated_pair(rv, rx, m, w3 + 3 * cv, w3 + 3 * cx);
        }
        slot = ws + r * L;
    } else {
        const float* hr = h + flat * L;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = load_pair(hr, (int64_t)(t + T1 * e) * L2 + m2);
        slot = ws + flat * L;
    }
#pragma unroll
    for (int e = 8; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
    fft_strided<L1, false, true>(v, t, tb.tw1, ColAcc{lds + c, Cfg::CP});
#pragma unroll
    for (int e = 0; e < 16; ++e) slot[(int64_t)(t + T1 * e) * L2 + m2] = v[e];
}

// Pass B: row FFTs over m2 (after the W_L^(k1*m2) twiddle), the pair step,
// then (MODE 0) the spectrum multiply, the inverse rows and the conjugate
// twiddle, in place; or (MODE 1) the scaled spectrum written in place.
// A unit is the row pair {p, L1-p} (p >= 1) or {0, L1/2} (p = 0).
template <int LOG1, int LOG2, int MODE>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::ROW_THREADS))
k_fs_row(float2* __restrict__ ws, const float2* __restrict__ spec, const float* __restrict__ bias, FsTables tb,
         int D, int o, int64_t row0) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T2 = Cfg::T2, U = Cfg::UNITS, RP = Cfg::RP;
    constexpr int64_t L = (int64_t)L1 * L2;
    constexpr int GROUPS = L1 / 2 / U;
    __shared__ float2 lds[2 * U * RP];
    const int ug = blockIdx.x % GROUPS;
    const int64_t r = blockIdx.x / GROUPS;
    const int64_t flat = row0 + r;
    const int tau = threadIdx.x;
    const int rho = tau / T2, t = tau % T2;
    const int p_row = ug * U + rho / 2;
    const int k1 = (rho & 1) == 0 ? p_row : (p_row == 0 ? L1 / 2 : L1 - p_row);
    float2* slot = (MODE == 0) ? ws + r * L : ws + flat * L;
    float2* rowp = slot + (int64_t)k1 * L2;
    const RowAcc racc{lds + rho * RP};

    float2 v[16], twv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int m2 = t + T2 * e;
        twv[e] = twiddle_L(tb, k1 * m2);
        v[e] = cmul(rowp[m2], twv[e]);
    }
    fft_strided<L2, false, false>(v, t, tb.tw2, racc);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) racc[t + T2 * e] = v[e];
    __syncthreads();

    // pair step: 2*T2 threads per unit, L2 pairs per unit
    const int unit = tau / (2 * T2), tp = tau % (2 * T2);
    const int p = ug * U + unit;
    const RowAcc aa{lds + (2 * unit) * RP};      // row p (or 0)
    const RowAcc ab{lds + (2 * unit + 1) * RP};  // row L1-p (or L1/2)
    const int k1a = p, k1b = (p == 0) ? L1 / 2 : L1 - p;
    int64_t d = 0;
    const float2* Hrow = nullptr;
    float bs = 0.f;
    if constexpr (MODE == 0) {
        d = flat % D;
        Hrow = spec + ((int64_t)o * D + d) * L;
        bs = bias[(int64_t)o * D + d] * (1.0f / (4.0f * (float)L));
    }
    const float sc = 1.0f / (8.0f * (float)L);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k2 = tp + 2 * T2 * e;
        if (p != 0) {
            // k = p + L1*k2 pairs with L - k = (L1-p) + L1*(L2-1-k2)
            const int ia = k2, ib = L2 - 1 - k2;
            const float2 w = cmul(tb.pa[p], tb.pb[k2]);
            if constexpr (MODE == 0) {
                float2 Yk, Ym;
                pair_conv(aa[ia], ab[ib], hadd(Hrow[(int64_t)k1a * L2 + ia], bs),
                          hadd(Hrow[(int64_t)k1b * L2 + ib], bs), w, Yk, Ym);
                aa[ia] = Yk;
                ab[ib] = Ym;
            } else {
                float2 Ak, Am;
                pair_unpack(aa[ia], ab[ib], w, Ak, Am);
                slot[(int64_t)k1a * L2 + ia] = fmul2(Ak, sc);
                slot[(int64_t)k1b * L2 + ib] = fmul2(Am, sc);
            }
        } else if (k2 == 0) {
            // k = 0 (with L) and k = L/2 (self-paired), both in row 0
            const float2 Z0 = aa[0];
            const float2 Zh = aa[L2 / 2];
            const float2 wh = tb.pb[L2 / 2];
            if constexpr (MODE == 0) {
                const float2 h0 = Hrow[0];
                float2 Yk, Ym;
                pair_conv(Z0, Z0, make_float2(h0.x + bs, 0.f), make_float2(h0.y + bs, 0.f), make_float2(1.f, 0.f),
                          Yk, Ym);
                aa[0] = Yk;
                const float2 Hh = hadd(Hrow[L2 / 2], bs);
                pair_conv(Zh, Zh, Hh, Hh, wh, Yk, Ym);
                aa[L2 / 2] = Yk;
            } else {
                float2 Ak, Am;
                pair_unpack(Z0, Z0, make_float2(1.f, 0.f), Ak, Am);
                slot[0] = make_float2(Ak.x * sc, Am.x * sc);
                pair_unpack(Zh, Zh, wh, Ak, Am);
                slot[L2 / 2] = fmul2(Ak, sc);
            }
        } else if (k2 < L2 / 2) {
            // row 0: k = L1*k2 pairs with L1*(L2-k2)
            const int ia = k2, ib = L2 - k2;
            const float2 w = tb.pb[k2];
            if constexpr (MODE == 0) {
                float2 Yk, Ym;
                pair_conv(aa[ia], aa[ib], hadd(Hrow[ia], bs), hadd(Hrow[ib], bs), w, Yk, Ym);
                aa[ia] = Yk;
                aa[ib] = Ym;
            } else {
                float2 Ak, Am;
                pair_unpack(aa[ia], aa[ib], w, Ak, Am);
                slot[ia] = fmul2(Ak, sc);
                slot[ib] = fmul2(Am, sc);
            }
        } else {
            // row L1/2: k = L1/2 + L1*j pairs with L1/2 + L1*(L2-1-j)
            const int j = k2 - L2 / 2;
            const int ia = j, ib = L2 - 1 - j;
            const float2 w = cmul(tb.pa[L1 / 2], tb.pb[j]);
            if constexpr (MODE == 0) {
                float2 Yk, Ym;
                pair_conv(ab[ia], ab[ib], hadd(Hrow[(int64_t)k1b * L2 + ia], bs),
                          hadd(Hrow[(int64_t)k1b * L2 + ib], bs), w, Yk, Ym);
                ab[ia] = Yk;
                ab[ib] = Ym;
            } else {
                float2 Ak, Am;
                pair_unpack(ab[ia], ab[ib], w, Ak, Am);
                slot[(int64_t)k1b * L2 + ia] = fmul2(Ak, sc);
                slot[(int64_t)k1b * L2 + ib] = fmul2(Am, sc);
            }
        }
    }
    if constexpr (MODE == 0) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = racc[t + T2 * e];
        fft_strided<L2, true, false>(v, t, tb.tw2, racc);
#pragma unroll
        for (int e = 0; e < 16; ++e) rowp[t + T2 * e] = cmulc(v[e], twv[e]);
    }
}

// Pass C: inverse column FFTs over k1, then the gate. The last step stores y;
// otherwise the gated result is the next step's input and its forward column
// FFTs (pass A of step o+1) run here, written back in place.
template <int LOG1, int LOG2, class TIO, bool LAST>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::COL_THREADS))
k_fs_colinv(float2* __restrict__ ws, const TIO* __restrict__ u, const float* __restrict__ w3, TIO* __restrict__ y,
            FsTables tb, int D, int N, int o, int64_t row0) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T1 = Cfg::T1, CB = Cfg::CB;
    constexpr int64_t L = (int64_t)L1 * L2;
    __shared__ float2 lds[L1 * Cfg::CP];
    const int cb = blockIdx.x % (L2 / CB);
    const int64_t r = blockIdx.x / (L2 / CB);
    const int64_t flat = row0 + r;
    const int64_t b = flat / D, d = flat % D;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m2 = cb * CB + c;
    float2* slot = ws + r * L;
    const ColAcc cacc{lds + c, Cfg::CP};
    float2 v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = slot[(int64_t)(t + T1 * e) * L2 + m2];
    fft_strided<L1, true, false>(v, t, tb.tw1, cacc);
    const int64_t C = (int64_t)(N + 1) * D;
    const int64_t cg = (int64_t)(LAST ? 0 : N - 2 - o) * D + d;
    const TIO* rg = u + (b * C + cg) * L;
    const float* wg = w3 + 3 * cg;
    if constexpr (LAST) {
        TIO* yr = y + (b * D + d) * L;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t m = (int64_t)(t + T1 * e) * L2 + m2;
            store_pair(yr, m, emul(v[e], conv3_pair(rg, m, wg[0], wg[1], wg[2])));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t m = (int64_t)(t + T1 * e) * L2 + m2;
            v[e] = emul(v[e], conv3_pair(rg, m, wg[0], wg[1], wg[2]));
        }
#pragma unroll
        for (int e = 8; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
        fft_strided<L1, false, true>(v, t, tb.tw1, cacc);
#pragma unroll
        for (int e = 0; e < 16; ++e) slot[(int64_t)(t + T1 * e) * L2 + m2] = v[e];
    }
}

// ================================================================== launchers

template <int LOGL>
static hipError_t launch_lds_forward_t(const LdsArgs& a, hipStream_t st) {
    constexpr int T = LdsCfg<LOGL>::THREADS;
    const int dgroups = (a.D + 7) / 8;
    const unsigned grid = (unsigned)(a.B * 8 * dgroups);
    if (a.bf16)
        hipLaunchKernelGGL((k_lds_forward<LOGL, uint16_t>), dim3(grid), dim3(T), 0, st, (const uint16_t*)a.u, a.w3,
                           a.spec, a.bias, (uint16_t*)a.y, a.tw, a.wpair, a.B, a.D, a.N);
    else
        hipLaunchKernelGGL((k_lds_forward<LOGL, float>), dim3(grid), dim3(T), 0, st, (const float*)a.u, a.w3,
                           a.spec, a.bias, (float*)a.y, a.tw, a.wpair, a.B, a.D, a.N);
    return hipGetLastError();
}

template <int LOGL>
static hipError_t launch_lds_spectrum_t(const float* h, float2* spec, int64_t rows, const float2* tw,
                                        const float2* wpair, hipStream_t st) {
    hipLaunchKernelGGL((k_lds_spectrum<LOGL>), dim3((unsigned)rows), dim3(LdsCfg<LOGL>::THREADS), 0, st, h, spec,
                       tw, wpair);
    return hipGetLastError();
}

hipError_t launch_lds_forward(int logL, const LdsArgs& a, hipStream_t st) {
    switch (logL) {
        case 4: return launch_lds_forward_t<4>(a, st);
        case 5: return launch_lds_forward_t<5>(a, st);
        case 6: return launch_lds_forward_t<6>(a, st);
        case 7: return launch_lds_forward_t<7>(a, st);
        case 8: return launch_lds_forward_t<8>(a, st);
        case 9: return launch_lds_forward_t<9>(a, st);
        case 10: return launch_lds_forward_t<10>(a, st);
        case 11: return launch_lds_forward_t<11>(a, st);
        case 12: return launch_lds_forward_t<12>(a, st);
        case 13: return launch_lds_forward_t<13>(a, st);
        case 14: return launch_lds_forward_t<14>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_lds_spectrum(int logL, const float* h, float2* spec, int64_t rows, const float2* tw,
                               const float2* wpair, hipStream_t st) {
    switch (logL) {
        case 4: return launch_lds_spectrum_t<4>(h, spec, rows, tw, wpair, st);
        case 5: return launch_lds_spectrum_t<5>(h, spec, rows, tw, wpair, st);
        case 6: return launch_lds_spectrum_t<6>(h, spec, rows, tw, wpair, st);
        case 7: return launch_lds_spectrum_t<7>(h, spec, rows, tw, wpair, st);
        case 8: return launch_lds_spectrum_t<8>(h, spec, rows, tw, wpair, st);
        case 9: return launch_lds_spectrum_t<9>(h, spec, rows, tw, wpair, st);
        case 10: return launch_lds_spectrum_t<10>(h, spec, rows, tw, wpair, st);
        case 11: return launch_lds_spectrum_t<11>(h, spec, rows, tw, wpair, st);
        case 12: return launch_lds_spectrum_t<12>(h, spec, rows, tw, wpair, st);
        case 13: return launch_lds_spectrum_t<13>(h, spec, rows, tw, wpair, st);
        case 14: return launch_lds_spectrum_t<14>(h, spec, rows, tw, wpair, st);
        default: return hipErrorInvalidValue;
    }
}

// Launches the passes of one chunk of rows. With `marks`, an event is recorded
// before the first launch and after every launch (1 + 2*(N-1) launches).
template <int LOG1, int LOG2>
static hipError_t fs_forward_chunk(const FsArgs& a, int64_t row0, int64_t nrows, hipStream_t st,
                                   hipEvent_t* marks) {
    using Cfg = FsCfg<LOG1, LOG2>;
    int mi = 0;
    auto mark = [&]() {
        if (marks) (void)hipEventRecord(marks[mi++], st);
    };
    mark();
    const unsigned gcol = (unsigned)(nrows * (Cfg::L2 / Cfg::CB));
    const unsigned grow = (unsigned)(nrows * (Cfg::L1 / 2 / Cfg::UNITS));
    const dim3 bcol(Cfg::COL_THREADS), brow(Cfg::ROW_THREADS);
    if (a.bf16)
        hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, uint16_t, 0>), dim3(gcol), bcol, 0, st, (const uint16_t*)a.u,
                           a.w3, (const float*)nullptr, a.ws, a.tb, a.D, a.N, row0);
    else
        hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, float, 0>), dim3(gcol), bcol, 0, st, (const float*)a.u, a.w3,
                           (const float*)nullptr, a.ws, a.tb, a.D, a.N, row0);
    mark();
    for (int o = 0; o < a.N - 1; ++o) {
        hipLaunchKernelGGL((k_fs_row<LOG1, LOG2, 0>), dim3(grow), brow, 0, st, a.ws, a.spec, a.bias, a.tb, a.D, o,
                           row0);
        mark();
        const bool last = (o == a.N - 2);
        if (a.bf16) {
            if (last)
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, uint16_t, true>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const uint16_t*)a.u, a.w3, (uint16_t*)a.y, a.tb, a.D, a.N, o, row0);
            else
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, uint16_t, false>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const uint16_t*)a.u, a.w3, (uint16_t*)a.y, a.tb, a.D, a.N, o, row0);
        } else {
            if (last)
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, float, true>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const float*)a.u, a.w3, (float*)a.y, a.tb, a.D, a.N, o, row0);
            else
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, float, false>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const float*)a.u, a.w3, (float*)a.y, a.tb, a.D, a.N, o, row0);
        }
        mark();
    }
    return hipGetLastError();
}

template <int LOG1, int LOG2>
static hipError_t fs_spectrum_t(const float* h, float2* spec, int64_t rows, const FsTables& tb, hipStream_t st) {
    using Cfg = FsCfg<LOG1, LOG2>;
    const unsigned gcol = (unsigned)(rows * (Cfg::L2 / Cfg::CB));
    const unsigned grow = (unsigned)(rows * (Cfg::L1 / 2 / Cfg::UNITS));
    hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, float, 1>), dim3(gcol), dim3(Cfg::COL_THREADS), 0, st,
                       (const float*)nullptr, (const float*)nullptr, h, spec, tb, 1, 2, (int64_t)0);
    hipLaunchKernelGGL((k_fs_row<LOG1, LOG2, 1>), dim3(grow), dim3(Cfg::ROW_THREADS), 0, st, spec,
                       (const float2*)nullptr, (const float*)nullptr, tb, 1, 0, (int64_t)0);
    return hipGetLastError();
}

#define HY_FS_CASES(X)                                                                                    \
    X(8, 4, 4) X(9, 4, 5) X(10, 5, 5) X(11, 5, 6) X(12, 6, 6) X(13, 6, 7) X(14, 7, 7) X(15, 7, 8) X(16, 8, 8) \
        X(17, 8, 9) X(18, 9, 9) X(19, 9, 10) X(20, 9, 11)

void fs_split(int logL, int* log1, int* log2) {
    int l1 = logL / 2;
    if (l1 > 9) l1 = 9;
    *log1 = l1;
    *log2 = logL - l1;
}

hipError_t launch_fs_forward_chunk(int logL, const FsArgs& a, int64_t row0, int64_t nrows, hipStream_t st,
                                   hipEvent_t* marks) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: return fs_forward_chunk<A, B>(a, row0, nrows, st, marks);
        HY_FS_CASES(X)
#undef X
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fs_spectrum(int logL, const float* h, float2* spec, int64_t rows, const FsTables& tb,
                              hipStream_t st) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: return fs_spectrum_t<A, B>(h, spec, rows, tb, st);
        HY_FS_CASES(X)
#undef X
        default: return hipErrorInvalidValue;
    }
}

int fs_row_units(int logL) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: return FsCfg<A, B>::UNITS;
        HY_FS_CASES(X)
#undef X
        default: return 0;
    }
}

}  // namespace hy
